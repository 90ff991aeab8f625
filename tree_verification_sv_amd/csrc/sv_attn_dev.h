// Device code of the ancestor-masked tree attention shared by sv_attention.hip
// (the sv_tree_attention kernels) and sv_step.hip (the one-launch verification
// step): LDS helpers, the per-sequence data checks, and the step's attention and
// merge roles.
//
// "EAGLE-Pangu: Accelerator-Safe Tree Speculative Decoding on Ascend NPUs",
// technical summary sec. 2 ("Ejecucion del Maestro con Mascara de Arbol
// Fusionada"): each draft token attends to the committed prefix, to its
// ancestors and to itself.  In the one-launch step the ancestor sets are derived
// from the parent array inside the launch ("Semantica de Tensores de Arbol
// Segura": the same walk and checks as sv_build_tree_mask), so no mask launch
// precedes the attention.
#pragma once
#include <float.h>
#include <math.h>

#include <type_traits>

#include "sv_mask_dev.h"

namespace {

constexpr float LOG2E = 1.4426950408889634f;

__device__ __forceinline__ int clamp_len(int L, int cap) { return L < 0 ? 0 : (L > cap ? cap : L); }

// Data checks behind the optional status array, run by one work-group per
// sequence: 6 when prefix_len lies outside [0, capacity] (it is clamped), 5 when
// a needed block-table entry is the ghost block 0 or outside the pool (read as
// the ghost block).
__device__ __forceinline__ void write_seq_status(const sv_attn_args& a, int b, int cap) {
  __shared__ int s_code;
  if (threadIdx.x == 0) s_code = 0;
  __syncthreads();
  const int L0 = a.prefix_len[b];
  if (L0 < 0 || L0 > cap) {
    if (threadIdx.x == 0) s_code = SV_SEQ_CAPACITY;
  } else if (a.paged) {
    // with the tree rows resident in the cache, positions L0 .. L0 + N - 1 are read too
    const int nblk = (L0 + (a.tree_in_cache ? a.N : 0) + a.block_size - 1) / a.block_size;
    for (int k = threadIdx.x; k < nblk; k += blockDim.x) {
      const int id = a.block_table[(int64_t)b * a.max_blocks + k];
      if (id < 1 || id >= a.num_blocks) atomicOr(&s_code, SV_SEQ_BLOCK);
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) a.status[b] = s_code;
}

typedef __attribute__((address_space(3))) void lds_void;

// 32-bit LDS address of a pointer into a __shared__ array
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
// Transposing 8-byte LDS reads (ds_read_b64_tr_b16): in every 16-lane group,
// lane 4q+e receives element e of the 8-byte pieces addressed by lanes q, 4+q,
// 8+q and 12+q.  Written as inline assembly: through the builtin, the compiler
// cannot tell these reads from the tile buffer that is still being filled by
// direct global->LDS loads and would wait for those loads as well.
// Four transposing reads (two d-blocks, low and high 8 keys) issued without waiting;
// tr_wait<N> must run before the values are used: it waits until at most N LDS
// operations are outstanding, and ties the registers to that point so that the
// compiler neither reads nor moves them earlier.
__device__ __forceinline__ void tr_read_issue(uint2 (&lo)[2], uint2 (&hi)[2], const uint32_t (&alo)[2],
                                              const uint32_t (&ahi)[2]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %4\n\tds_read_b64_tr_b16 %1, %5\n\t"
      "ds_read_b64_tr_b16 %2, %6\n\tds_read_b64_tr_b16 %3, %7"
      : "=&v"(lo[0]), "=&v"(hi[0]), "=&v"(lo[1]), "=&v"(hi[1])
      : "v"(alo[0]), "v"(ahi[0]), "v"(alo[1]), "v"(ahi[1])
      : "memory");
}
template <int N>
__device__ __forceinline__ void tr_wait(uint2 (&lo)[2], uint2 (&hi)[2]) {
  asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(lo[0]), "+v"(hi[0]), "+v"(lo[1]), "+v"(hi[1]) : "n"(N) : "memory");
}

// x combined with the same lane of the other 32-lane half of the wave, through one
// v_permlane32_swap (no LDS round trip): every lane gets op(x[l], x[l ^ 32])
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Split partials that a merge work-group of the same launch reads are written and read with
// relaxed device-scope atomic 64-bit accesses (coherent across the XCDs' caches); the writer
// waits for its stores to complete before it counts in, and the merge loads them only after
// it has seen every split's count.  No cache write-back or invalidation is needed.
__device__ __forceinline__ void st_dev64(void* p, uint64_t v) {
  __hip_atomic_store((uint64_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_dev64(const void* p) {
  return __hip_atomic_load((uint64_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------------ MFMA attention
constexpr uint32_t AT_SPIN_LIMIT = 1u << 22;  // bounded wait of a merge work-group of the one-launch step (polls)
constexpr int MF_WAVES = 8;                // waves of the MFMA kernel (two per SIMD)
constexpr int MF_THREADS = 64 * MF_WAVES;
constexpr int MF_QB = 1;                   // 32-row query blocks per wave
constexpr int KT = 64;  // keys per tile
constexpr float AT_LAZY = 8.f;  // log2 of the largest weight before the reference maximum moves
constexpr int AT_NT = 2;        // cache policy of the K/V tile loads: non-temporal

struct AttnPlan {
  int32_t G, M, QB, QT, qtiles, nsplit, chunk, ntt, W, cap;
  float cscale;  // scale * log2(e)
  uint32_t pool_bytes;  // paged: bytes of one K (or V) pool, < 4 GiB
  uint16_t* opart;  // [units][nsplit][QT][D] bf16: the split's output row O / l
  float* mlpart;    // [units][nsplit][QT][2]: running max (scaled by log2 e) and l
  // one-launch step only: splits count in on arrive[unit] after their partials (release),
  // and mper merge work-groups of mrows output rows each combine a (sequence, KV head) pair
  uint32_t* arrive;
  int32_t nunits, nwg, mrows, mper;
};

// One 64-key tile in LDS: K rows then V rows, row-major without padding.  The
// 16-byte chunks of row r are stored XOR-swizzled (global chunk c sits in slot
// c ^ swz(r)), which keeps both the 16-byte K fragment reads and the 8-byte
// transposing V reads free of bank conflicts.  Tiles are written by direct
// global -> LDS loads (each load instruction of a wave fills 1 KB: lane l's 16
// bytes land at byte 16 l), so staging a tile costs no registers.
template <int D>
struct Tile {
  static constexpr int KT = 64;
  static constexpr int CPR = D / 8;                   // 16-byte chunks per row
  static constexpr int ROWB = D * 2;                  // bytes per row
  static constexpr int RPI = 64 / CPR;                // rows filled by one load instruction
  static constexpr int IPW = KT / RPI / MF_WAVES;     // load instructions per wave per tensor
  static constexpr int RPW = RPI * IPW;               // rows filled by one wave
  static constexpr int TBYTES = KT * ROWB;            // one tensor of the tile
  static constexpr int BUF = 2 * TBYTES;              // K and V
  static constexpr int QROWS = 32 * MF_QB * MF_WAVES;  // query rows per work-group
  // Any 16 consecutive rows (8 row pairs for D = 64) take distinct slots, so the 16-lane groups
  // of a 16-byte fragment read hit every bank once; and each aligned group of 4 rows differs in
  // bits 2-3 of the slot, so the 32-lane groups of an 8-byte transposing V read (4 rows x 4
  // chunks x 2 halves) do too.
  __device__ static __forceinline__ int swz(int r) {
    return CPR == 16 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
  }
};

// Ancestor bitsets of every node of sequence b into LDS (anc[i * 4 + w], four words per node),
// by the rule of sv_build_tree_mask: walk up at most max_depth nodes; a parent out of range,
// a revisited node or a path longer than max_depth makes the node invalid, and an invalid node
// sees only itself.  spar: N ints of LDS.  Every thread of the work-group calls it.
__device__ __forceinline__ void step_ancestors(const int32_t* __restrict__ parents, int b, int N, int max_depth,
                                               int32_t* spar, uint64_t* anc) {
  const int t = threadIdx.x;
  for (int i = t; i < N; i += blockDim.x) spar[i] = parents[(int64_t)b * N + i];
  __syncthreads();
  for (int i = t; i < N; i += blockDim.x) {
    uint64_t bits[SV_MAX_W] = {0, 0, 0, 0};
    bit_set(bits, i);
    int count = 1, cur = i;
    bool ok = true;
    for (int step = 0; step <= SV_MAX_DEPTH; ++step) {  // every iteration exits or grows count
      const int pp = spar[cur];
      if (pp < -1 || pp >= N) { ok = false; break; }
      if (pp == -1) break;
      if (bit_get(bits, pp)) { ok = false; break; }
      if (count + 1 > max_depth) { ok = false; break; }
      bit_set(bits, pp);
      ++count;
      cur = pp;
    }
    if (!ok) {  // an invalid node sees only itself
      bits[0] = bits[1] = bits[2] = bits[3] = 0;
      bit_set(bits, i);
    }
#pragma unroll
    for (int w = 0; w < SV_MAX_W; ++w) anc[i * 4 + w] = bits[w];
  }
  __syncthreads();
}

// The work of one attention work-group (logical index lid, MF_THREADS threads): see the file
// comment of sv_attention.hip.  kvA, kvB: the two K/V tile buffers and qsb: the query rows,
// three separate LDS arrays (so that the direct loads into one are known not to alias the
// reads of another).  derive_parents (nullable): the ancestor sets of the query nodes are
// derived from this parent array into aux (>= 9 KB of LDS) by the rule of sv_build_tree_mask
// instead of being read from a.anc_bits.  p.arrive (nullable): after writing its partial the
// work-group counts in on its unit's counter with a release.  bt_lds (nullable, AT_BT_MAX
// entries of LDS): on the paged path the block ids of the work-group's key range are read into
// it once, so that no tile load waits for a block-table read.  Every thread calls it.
constexpr int AT_BT_MAX = 512;  // block ids held in LDS: key ranges of up to 8192 tokens
template <int D>
__device__ __forceinline__ void attn_mfma_body(const sv_attn_args& a, const AttnPlan& p, int lid, unsigned char* kvA,
                                               unsigned char* kvB, unsigned char* qsb,
                                               const int32_t* __restrict__ derive_parents, int max_depth,
                                               unsigned char* aux, int32_t* bt_lds = nullptr) {
  using TL = Tile<D>;
  constexpr int QB = MF_QB;             // 32-row query blocks per wave
  constexpr int KT64 = TL::KT;
  constexpr int DS = D / 16;            // 16-wide k-steps of S = K Q^T
  constexpr int DB = D / 32;            // 32-wide d-blocks of O^T
  constexpr uint32_t ROWB = TL::ROWB;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);  // uniform wave index
  const int lq = lane & 31;  // query column / key row inside a 32-block
  const int hf = lane >> 5;  // which half of the k dimension this lane feeds
  // the two waves sharing a SIMD get different issue priorities, so that one runs ahead
  // of the other inside each tile and its softmax overlaps the other's MFMAs
  if (w < MF_WAVES / 2) __builtin_amdgcn_s_setprio(1);

  const int qtile = lid % p.qtiles;
  const int split = (lid / p.qtiles) % p.nsplit;
  const int pair = lid / (p.qtiles * p.nsplit);
  const int b = pair / a.Hkv;
  const int g = pair % a.Hkv;
  const int N = a.N, Hq = a.Hq, G = p.G;

  if (a.status && g == 0 && qtile == 0 && split == 0) write_seq_status(a, b, p.cap);
  const int L = clamp_len(a.prefix_len[b], p.cap);
  const int k0 = split * p.chunk;
  const int k1 = min(k0 + p.chunk, L);
  const int ntp = k1 > k0 ? (k1 - k0 + KT64 - 1) / KT64 : 0;
  const bool last = split == p.nsplit - 1;
  const int ntt = last ? p.ntt : 0;
  const int ntiles = ntp + ntt;

  // rows of this wave: m = qtile * QT + w * 32 QB + qb * 32 + lq
  const int mw = qtile * p.QT + w * 32 * QB;
  const bool active = mw < p.M;  // uniform: the wave has at least one valid query row

  const __bf16* qg = (const __bf16*)a.q;
  const uint16_t* kc = (const uint16_t*)a.k_cache;
  const uint16_t* vc = (const uint16_t*)a.v_cache;
  const uint16_t* kt = (const uint16_t*)a.k_tree;
  const uint16_t* vt = (const uint16_t*)a.v_tree;

  // ---- tile loads: wave w fills rows RPW w .. RPW w + RPW - 1 of K and of V.  Keys past
  // the valid range are clamped onto the last valid key of the tile (finite data,
  // masked out of the softmax), so no load ever leaves the tensor.
  const int64_t plane = (int64_t)b * a.Hkv + g;
  // tree rows: the separate tree K/V rows 1..N, or (tree_in_cache) cache positions
  // L .. L + N - 1 of this sequence; L <= capacity - N, so they lie inside the cache
  const bool tic = a.tree_in_cache != 0;
  const bool tic_paged = tic && a.paged;
  __amdgpu_buffer_rsrc_t rk, rv, rkt, rvt;
  if (a.paged) {
    rk = __builtin_amdgcn_make_buffer_rsrc((void*)kc, 0, (int)p.pool_bytes, 0x00020000);
    rv = __builtin_amdgcn_make_buffer_rsrc((void*)vc, 0, (int)p.pool_bytes, 0x00020000);
  } else {
    rk = __builtin_amdgcn_make_buffer_rsrc((void*)(kc + plane * a.Lcap * D), 0, (int)(a.Lcap * ROWB), 0x00020000);
    rv = __builtin_amdgcn_make_buffer_rsrc((void*)(vc + plane * a.Lcap * D), 0, (int)(a.Lcap * ROWB), 0x00020000);
  }
  if (tic_paged) {
    rkt = rk;  // rows gathered through the block table, lane by lane
    rvt = rv;
  } else if (tic) {
    rkt = __builtin_amdgcn_make_buffer_rsrc((void*)(kc + (plane * a.Lcap + L) * D), 0, (int)(N * ROWB), 0x00020000);
    rvt = __builtin_amdgcn_make_buffer_rsrc((void*)(vc + (plane * a.Lcap + L) * D), 0, (int)(N * ROWB), 0x00020000);
  } else {
    rkt = __builtin_amdgcn_make_buffer_rsrc((void*)(kt + (plane * (N + 1) + 1) * D), 0, (int)(N * ROWB), 0x00020000);
    rvt = __builtin_amdgcn_make_buffer_rsrc((void*)(vt + (plane * (N + 1) + 1) * D), 0, (int)(N * ROWB), 0x00020000);
  }
  // paged prefix: the block ids of blocks bt0 .. of the key range, sanitised, into LDS
  int bt0 = 0;
  bool bt_pre = false;
  if (a.paged && bt_lds && ntp > 0) {
    bt0 = k0 / 16;
    const int nbk = (k1 - 1) / 16 - bt0 + 1;
    if (nbk <= AT_BT_MAX) {  // uniform
      for (int i = t; i < nbk; i += MF_THREADS) {
        const int id = a.block_table[(int64_t)b * a.max_blocks + bt0 + i];
        bt_lds[i] = (id < 0 || id >= a.num_blocks) ? 0 : id;
      }
      __syncthreads();
      bt_pre = true;
    }
  }
  auto load_tile = [&](int tile, unsigned char* kb) {
    const bool tree = tile >= ntp;
    int klast;
    int t0 = 0;
    uint32_t soff = 0;
    if (tree) {
      t0 = (tile - ntp) * KT64;
      klast = min(KT64, N - t0) - 1;
      soff = tic_paged ? 0u : (uint32_t)t0 * ROWB;
    } else {
      const int j0 = k0 + tile * KT64;
      klast = min(KT64, k1 - j0) - 1;
      if (a.paged) {
        // the wave's rows lie in one 16-token block (RPW divides 16); past the end the
        // clamped key min(r, klast) = klast, so its block is the one used
        const int blk = (j0 + min(TL::RPW * w, klast)) / 16;
        int id;
        if (bt_pre) {
          id = __builtin_amdgcn_readfirstlane(bt_lds[blk - bt0]);
        } else {
          id = __builtin_amdgcn_readfirstlane(a.block_table[(int64_t)b * a.max_blocks + blk]);
          id = (id < 0 || id >= a.num_blocks) ? 0 : id;
        }
        soff = (uint32_t)(((int64_t)id * a.Hkv + g) * 16) * ROWB;
      } else {
        soff = (uint32_t)j0 * ROWB;
      }
    }
    const bool paged_tile = !tree && a.paged;
    const __amdgpu_buffer_rsrc_t rK = tree ? rkt : rk;
    const __amdgpu_buffer_rsrc_t rV = tree ? rvt : rv;
#pragma unroll
    for (int it = 0; it < TL::IPW; ++it) {
      const int n = w * TL::IPW + it;                    // 1-KB piece of the tile (uniform)
      const int r = n * TL::RPI + lane / TL::CPR;        // row this lane fills
      const int c = (lane % TL::CPR) ^ TL::swz(r);       // global chunk stored in its slot
      const int key = min(r, klast);
      uint32_t off;
      if (tree && tic_paged) {
        // tree node t0 + key sits at logical position L + t0 + key < capacity
        const int pos = L + t0 + key;
        int id = a.block_table[(int64_t)b * a.max_blocks + pos / 16];
        id = (id < 0 || id >= a.num_blocks) ? 0 : id;
        off = (uint32_t)((((int64_t)id * a.Hkv + g) * 16 + (pos & 15)) * ROWB + c * 16);
      } else {
        off = (uint32_t)((paged_tile ? (key & 15) : key) * ROWB + c * 16);
      }
      // non-temporal: each K/V row is read by one work-group once (the query rows, read by every
      // split of a pair, keep the default policy)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rK, (lds_void*)(kb + n * 1024), 16, off, soff, 0, AT_NT);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rV, (lds_void*)(kb + TL::TBYTES + n * 1024), 16, off, soff, 0, AT_NT);
    }
  };

  if (0 < ntiles) load_tile(0, kvA);

  // ---- the work-group's query rows into LDS, swizzled like K (rows past M repeat row
  // M - 1; their outputs are never written).  The B operand of S^T = K Q^T for lane
  // (lq, hf) and k-step ds is Q row lq, d = 16*ds + 8*hf .. +7.
  {
    constexpr int NQ = TL::QROWS * TL::CPR / 64 / MF_WAVES;  // 1-KB pieces per wave
#pragma unroll
    for (int it = 0; it < NQ; ++it) {
      const int n = w * NQ + it;
      const int r = n * TL::RPI + lane / TL::CPR;
      const int c = (lane % TL::CPR) ^ TL::swz(r);
      const int m = min(qtile * p.QT + r, p.M - 1);
      const int node = m / G, h = g * G + m % G;
      __builtin_amdgcn_global_load_lds((const void*)(qg + (((int64_t)b * N + node) * Hq + h) * D + c * 8),
                                       (lds_void*)(qsb + n * 1024), 16, 0, 0);
    }
  }
  // the last split reads the tree keys: in the one-launch step their masks come from the
  // parent array, derived here into LDS
  const uint64_t* anc_lds = nullptr;
  if (derive_parents && ntt > 0) {
    step_ancestors(derive_parents, b, N, max_depth, (int32_t*)(aux + SV_MAX_N * 4 * 8), (uint64_t*)aux);
    anc_lds = (const uint64_t*)aux;
  }
  int qnode[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int m = mw + qb * 32 + lq;
    qnode[qb] = m < p.M ? m / G : -1;
  }

  sv_f32x16 oacc[QB][DB];
  float mrun[QB], lrun[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    mrun[qb] = -INFINITY;
    lrun[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[qb][db][r] = 0.f;
  }

  // lane-constant parts of the LDS fragment reads
  const int k_off = lq * ROWB;                       // K row lq of a 32-key block (+ 32 kb rows)
  const int k_swz = TL::swz(lq);
  // transposing V reads: source lane (16 u + 4 j + q) addresses row 4 (u / 2) + j (+ 8 for
  // the upper half) at element column 16 (u % 2) + 4 q, i.e. chunk 2 (u % 2) + q / 2, half q % 2
  const int tr_row = 4 * (lane >> 5) + ((lane & 15) >> 2);
  const int tr_chunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int tr_half = (lane & 1) * 8;
  const int tr_swz_lo = TL::swz(tr_row), tr_swz_hi = TL::swz(tr_row + 8);

  auto compute = [&](int tile, const unsigned char* Kb) {
    const unsigned char* Vb = Kb + TL::TBYTES;
    const bool tree = tile >= ntp;
    const int j0 = k0 + tile * KT64;
    const int t0 = (tile - ntp) * KT64;

    // ---- S^T = K Q^T for two 32-key blocks
    sv_f32x16 sacc[QB][2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[qb][kb][r] = 0.f;
    // the fragments of k-steps ds + 1 and ds + 2 are read while the MFMAs of step ds run, so
    // the LDS latency is hidden behind them
    sv_bf16x8 qf[3][QB], kf[3][2];
    auto frag = [&](int ds, int buf) {
      const int kslot = ((2 * ds + hf) ^ k_swz) * 16;  // Q and K rows share the swizzle of row lq
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        qf[buf][qb] = *(const sv_bf16x8*)(qsb + (w * 32 * QB + qb * 32) * ROWB + k_off + kslot);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) kf[buf][kb] = *(const sv_bf16x8*)(Kb + kb * 32 * ROWB + k_off + kslot);
    };
    frag(0, 0);
    frag(1, 1);
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      if (ds + 2 < DS) frag(ds + 2, (ds + 2) % 3);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          sacc[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ds % 3][kb], qf[ds % 3][qb], sacc[qb][kb], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);  // one step in flight at a time (register pressure)
    }

    __builtin_amdgcn_sched_barrier(0);
    // ---- masks + online softmax (lane owns query column lq; keys 32 kb + 8 (r/4) + 4 hf + r%4)
    const bool full = !tree && (j0 + KT64 <= k1);
    sv_bf16x8 pf[QB][2][2];
    bool moved = false;
    float alpha[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      // scores stay unscaled here; the scale (times log2 e) is folded into the exponent
      if (!full && !tree) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kk = 32 * kb + 8 * (r >> 2) + 4 * hf + (r & 3);
            if (j0 + kk >= k1) sacc[qb][kb][r] = -INFINITY;
          }
      } else if (tree) {
        const int wi = t0 >> 6;  // uniform: the tile is one 64-bit mask word of the query node's bitset
        uint64_t aw = qnode[qb] < 0 ? 0ull
                      : (anc_lds ? anc_lds[qnode[qb] * 4 + wi] : a.anc_bits[((int64_t)b * N + qnode[qb]) * p.W + wi]);
        const int lim = N - t0;  // keys of the tile that are tree nodes
        if (lim < 64) aw &= (1ull << lim) - 1ull;
        // shift this lane's key half to bit 0, so every register tests a constant bit
        const uint64_t sh = aw >> (4 * hf);
        const uint32_t a_lo = (uint32_t)sh, a_hi = (uint32_t)(sh >> 32);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const uint32_t word = kb == 0 ? a_lo : a_hi;
            if (((word >> (8 * (r >> 2) + (r & 3))) & 1u) == 0) sacc[qb][kb][r] = -INFINITY;
          }
      }
      // maximum over the lane's 32 scores in four independent chains, then across the two
      // halves of the wave (lanes l and l + 32 hold the two key halves of query column l)
      float mc[4] = {sacc[qb][0][0], sacc[qb][0][1], sacc[qb][0][2], sacc[qb][0][3]};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kb || r >= 4) mc[r & 3] = fmaxf(mc[r & 3], sacc[qb][kb][r]);
      float mt = halves_max(fmaxf(fmaxf(mc[0], mc[1]), fmaxf(mc[2], mc[3])));
      // The reference maximum moves only when a score exceeds it by more than 2^AT_LAZY in the
      // weights (or at the first visible score): the weights then stay below 2^AT_LAZY, exact in
      // bf16's range and in the fp32 sums, and most tiles skip the rescale of the accumulators.
      const bool up = mt * p.cscale > mrun[qb] * p.cscale + AT_LAZY;  // false while mt is -inf
      const float mnew = up ? mt : mrun[qb];
      const float ms = mnew == -INFINITY ? 0.f : mnew * p.cscale;  // nothing visible yet: weights stay 0
      alpha[qb] = up ? __builtin_amdgcn_exp2f(mrun[qb] * p.cscale - ms) : 1.f;
      moved |= up;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          pf[qb][kb][r >> 3][r & 7] = (__bf16)__builtin_amdgcn_exp2f(fmaf(sacc[qb][kb][r], p.cscale, -ms));
      // the row sum of the bf16 weights the P V product uses: two per dot instruction
      float ps[4] = {0.f, 0.f, 0.f, 0.f};  // four independent chains
      const sv_bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
          const sv_bf16x8 v = pf[qb][kb][t2];
          ps[0] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 0, 1), one2, ps[0], false);
          ps[1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 2, 3), one2, ps[1], false);
          ps[2] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 4, 5), one2, ps[2], false);
          ps[3] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 6, 7), one2, ps[3], false);
        }
      const float psum = halves_sum((ps[0] + ps[1]) + (ps[2] + ps[3]));
      lrun[qb] = lrun[qb] * alpha[qb] + psum;
      mrun[qb] = mnew;
      __builtin_amdgcn_sched_barrier(0);  // one query block at a time (register pressure)
    }
    // rescale the accumulators only when some lane's running maximum moved
    if (__ballot(moved)) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[qb][db][r] *= alpha[qb];
    }

    __builtin_amdgcn_sched_barrier(0);
    // ---- O^T += V^T P^T; the 16-key step (kb, t2) holds keys 32 kb + 16 t2 + 4 hf + {0..3, 8..11}.
    // Half-steps of two d-blocks: the transposing reads of half-steps h + 1 and h + 2 are
    // issued before the MFMAs of half-step h, which wait only for their own reads (LDS reads
    // complete in order, so at most the 8 newer reads may still be outstanding).
    constexpr int NH = 2 * DB;  // 4 steps (kb, t2) x DB / 2 halves
    uint2 vlo[3][2], vhi[3][2];
    auto tr_issue = [&](int h, int buf) {
      const int st = h / (DB / 2), d0 = (h % (DB / 2)) * 2;  // step kb * 2 + t2, first d-block
      const int kb = st >> 1, t2 = st & 1;
      const uint32_t rlo = lds_addr(Vb) + (32 * kb + 16 * t2 + tr_row) * ROWB + tr_half;
      const uint32_t rhi = rlo + 8 * ROWB;
      uint32_t alo[2], ahi[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int c = 4 * (d0 + j) + tr_chunk;
        alo[j] = rlo + ((c ^ tr_swz_lo) << 4);
        ahi[j] = rhi + ((c ^ tr_swz_hi) << 4);
      }
      tr_read_issue(vlo[buf], vhi[buf], alo, ahi);
    };
    tr_issue(0, 0);
    tr_issue(1, 1);
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      const int buf = h % 3;
      if (h + 2 < NH) {
        tr_issue(h + 2, (h + 2) % 3);
        tr_wait<8>(vlo[buf], vhi[buf]);
      } else if (h + 1 < NH) {
        tr_wait<4>(vlo[buf], vhi[buf]);
      } else {
        tr_wait<0>(vlo[buf], vhi[buf]);
      }
      const int st = h / (DB / 2), d0 = (h % (DB / 2)) * 2;
      const int kb = st >> 1, t2 = st & 1;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const sv_bf16x8 vf = __builtin_bit_cast(sv_bf16x8, make_uint4(vlo[buf][j].x, vlo[buf][j].y, vhi[buf][j].x, vhi[buf][j].y));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          oacc[qb][d0 + j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[qb][kb][t2], oacc[qb][d0 + j], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- main loop: even tiles compute from kvA while the next tile streams into kvB, and back
  for (int tile = 0; tile < ntiles; tile += 2) {
    __builtin_amdgcn_s_waitcnt(0);  // this thread's loads of `tile` (and the Q rows) have landed
    __syncthreads();                // ... and everyone's; every wave is done with tile - 1
    if (tile + 1 < ntiles) load_tile(tile + 1, kvB);
    if (active) compute(tile, kvA);
    if (tile + 1 >= ntiles) break;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tile + 2 < ntiles) load_tile(tile + 2, kvA);
    if (active) compute(tile + 1, kvB);
  }
  // ---- write: bf16 output (single split) or per-split partials: the normalised row
  // O / l in bf16 and (m, l) in fp32.  The wave stages its rows in its own query rows of
  // LDS (no other wave reads them, and its own reads of them are done), swizzled like the
  // query layout, then stores whole rows with 16 consecutive bytes per lane.
  const int unit = pair * p.qtiles + qtile;
  const int64_t pidx = (int64_t)unit * p.nsplit + split;
  if (active) {
  unsigned char* ob = qsb + (w * 32 * QB) * ROWB;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int ql = w * 32 * QB + qb * 32 + lq;
    const int m = qtile * p.QT + ql;
    const float inv = lrun[qb] > 0.f ? 1.f / lrun[qb] : 0.f;
    if (p.nsplit > 1 && hf == 0 && m < p.M) {
      float* dst = p.mlpart + (pidx * p.QT + ql) * 2;
      if (p.arrive)  // read by a merge work-group of this launch
        st_dev64(dst, ((uint64_t)__float_as_uint(lrun[qb]) << 32) | __float_as_uint(mrun[qb] * p.cscale));
      else
        *(float2*)dst = make_float2(mrun[qb] * p.cscale, lrun[qb]);
    }
    const int sw = TL::swz(lq);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int c = 4 * db + rq;  // 16-byte chunk of elements db*32 + 8 rq .. + 7; this lane holds half hf
        const uint32_t w0 = f32_to_bf16_bits(oacc[qb][db][4 * rq + 0] * inv) |
                            ((uint32_t)f32_to_bf16_bits(oacc[qb][db][4 * rq + 1] * inv) << 16);
        const uint32_t w1 = f32_to_bf16_bits(oacc[qb][db][4 * rq + 2] * inv) |
                            ((uint32_t)f32_to_bf16_bits(oacc[qb][db][4 * rq + 3] * inv) << 16);
        *(uint2*)(ob + (qb * 32 + lq) * ROWB + ((c ^ sw) << 4) + 8 * hf) = make_uint2(w0, w1);
      }
  }
  constexpr int CPR = TL::CPR, RPO = 64 / CPR;  // 16-byte chunks per row, rows per store
#pragma unroll
  for (int i = 0; i < 32 * QB / RPO; ++i) {
    const int r = i * RPO + lane / CPR;  // row of the wave's block
    const int ch = lane % CPR;
    const uint4 v = *(const uint4*)(ob + r * ROWB + ((ch ^ TL::swz(r)) << 4));
    const int ql = w * 32 * QB + r;
    const int m = qtile * p.QT + ql;
    if (m < p.M) {
      uint16_t* orow = p.nsplit == 1 ? (uint16_t*)a.out + (((int64_t)b * N + m / G) * Hq + g * G + m % G) * D
                                     : p.opart + (pidx * p.QT + ql) * D;
      if (p.nsplit > 1 && p.arrive) {
        st_dev64(orow + ch * 8, ((uint64_t)v.y << 32) | v.x);
        st_dev64(orow + ch * 8 + 4, ((uint64_t)v.w << 32) | v.z);
      } else {
        *(uint4*)(orow + ch * 8) = v;
      }
    }
  }
  }  // active
  if (p.arrive && p.nsplit > 1) {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0);  // this thread's partial stores have completed
    asm volatile("" ::: "memory");
    __syncthreads();  // ... and every wave's, before the split counts in
    if (t == 0) __hip_atomic_fetch_add(&p.arrive[unit], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// One merge work-group of the step: output rows m0 .. m0 + mrows - 1 of one (sequence, KV head)
// pair.  It waits (bounded) until every split of the units those rows belong to has counted in,
// then combines the splits' normalised rows with weights exp2(m_s - max) l_s, as
// k_attn_combine does.  TPR threads per row, one 16-byte chunk each.  s_f: LDS for
// (TH / TPR) x 64 split weights.  On an expired wait the sequence's attention status is 7.
template <int D, int TH>
__device__ __forceinline__ void step_merge(const sv_attn_args& a, const AttnPlan& p, int mid, float* s_f) {
  constexpr int TPR = D / 8;                // threads per output row
  constexpr int RPP = TH / TPR;             // rows per pass
  constexpr int SB = 16;                    // split rows in flight per thread
  constexpr int MLN = 64 / TPR;             // (m, l) pairs per thread (at most 64 splits)
  const int t = threadIdx.x;
  const int pair = mid / p.mper, part = mid % p.mper;
  const int b = pair / a.Hkv, g = pair % a.Hkv;
  const int m0 = part * p.mrows;
  const int m1 = min(m0 + p.mrows, p.M);
  if (m0 >= m1) return;  // uniform
  __shared__ int s_late;
  if (t == 0) {
    int late = 0;
    for (int q = m0 / p.QT; q <= (m1 - 1) / p.QT; ++q) {
      uint32_t* cnt = &p.arrive[pair * p.qtiles + q];
      uint32_t spins = 0;
      while (__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < (uint32_t)p.nsplit) {
        if (++spins > AT_SPIN_LIMIT) { late = 1; break; }
        __builtin_amdgcn_s_sleep(1);
      }
    }
    s_late = late;
  }
  __syncthreads();
  if (s_late && a.status) atomicMax(&a.status[b], SV_SEQ_TIMEOUT);
  const int ns = p.nsplit;
  const int G = p.G;
  const int lr = t / TPR, c = t % TPR;
  for (int mb = m0; mb < m1; mb += RPP) {
    const int m = mb + lr;
    const bool on = m < m1;
    const int mm = on ? m : m1 - 1;
    const int unit = pair * p.qtiles + mm / p.QT, ql = mm % p.QT;
    // every load of the row goes out first (one memory round trip): thread c takes the (m, l) of
    // splits c, c + TPR, ... and its 16-byte chunk of the first SB splits' rows
    uint64_t mlw[MLN];
#pragma unroll
    for (int i = 0; i < MLN; ++i)
      mlw[i] = ld_dev64(p.mlpart + (((int64_t)unit * ns + min(c + i * TPR, ns - 1)) * p.QT + ql) * 2);
    uint4 part[SB];
    auto load_parts = [&](int s0) {
#pragma unroll
      for (int k = 0; k < SB; ++k) {
        const int s = min(s0 + k, ns - 1);
        const uint16_t* src = p.opart + (((int64_t)unit * ns + s) * p.QT + ql) * D + c * 8;
        const uint64_t lo = ld_dev64(src), hi = ld_dev64(src + 4);
        part[k] = make_uint4((uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32));
      }
    };
    load_parts(0);
    // weights exp2(m_s - max) l_s: max and sum over the row's lanes
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < MLN; ++i)
      if (c + i * TPR < ns) mx = fmaxf(mx, __uint_as_float((uint32_t)mlw[i]));
#pragma unroll
    for (int o = TPR / 2; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    float lsum = 0.f;
#pragma unroll
    for (int i = 0; i < MLN; ++i) {
      const int s = c + i * TPR;
      const float ms = __uint_as_float((uint32_t)mlw[i]), ls = __uint_as_float((uint32_t)(mlw[i] >> 32));
      const float f = ms == -INFINITY ? 0.f : exp2f(ms - mx) * ls;
      if (s < ns) {
        s_f[lr * 64 + s] = f;
        lsum += f;
      }
    }
#pragma unroll
    for (int o = TPR / 2; o > 0; o >>= 1) lsum += __shfl_xor(lsum, o);
    wave_lds_sync();  // the row's weights come from lanes of the same wave
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    for (int s0 = 0; s0 < ns; s0 += SB) {
      if (s0 > 0) load_parts(s0);
#pragma unroll
      for (int k = 0; k < SB; ++k) {
        const float f = s0 + k < ns ? s_f[lr * 64 + min(s0 + k, 63)] : 0.f;  // past the splits: weight 0
        const uint32_t ww[4] = {part[k].x, part[k].y, part[k].z, part[k].w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          acc[2 * h] = fmaf(f, __uint_as_float(ww[h] << 16), acc[2 * h]);
          acc[2 * h + 1] = fmaf(f, __uint_as_float(ww[h] & 0xffff0000u), acc[2 * h + 1]);
        }
      }
    }
    const float inv = (mx != -INFINITY && lsum > 0.f) ? 1.f / lsum : 0.f;
    if (on) {
      uint32_t o4[4];
#pragma unroll
      for (int h = 0; h < 4; ++h)
        o4[h] = f32_to_bf16_bits(acc[2 * h] * inv) | ((uint32_t)f32_to_bf16_bits(acc[2 * h + 1] * inv) << 16);
      const int node = m / G, hh = g * G + m % G;
      *(uint4*)((uint16_t*)a.out + (((int64_t)b * a.N + node) * a.Hq + hh) * D + c * 8) =
          make_uint4(o4[0], o4[1], o4[2], o4[3]);
    }
    wave_lds_sync();  // the weights are read before the next pass overwrites them
  }
}

}  // namespace
