// Ancestor-masked GQA tree attention over a contiguous or paged KV prefix.
//
// "EAGLE-Pangu: Accelerator-Safe Tree Speculative Decoding on Ascend NPUs",
// technical summary sec. 2 ("Ejecucion del Maestro con Mascara de Arbol
// Fusionada"): each draft token attends to the committed prefix, to its
// ancestors and to itself, never to other branches.  "Accelerating Sonar
// Through Speculation", section "EAGLE": a custom mask over the whole
// sequence costs attention speed, so here the prefix block is dense and
// mask-free and only the N x N tree block reads the per-node ancestor bitsets.
//
// Kernels
//  k_attn_mfma<D>  bf16, the hot path.  A work-group owns one KV head g of one
//     sequence, a tile of up to 256 query rows (row m = node*G + head in group,
//     so the G query heads that share a KV head form one dense contraction of
//     M = N*G rows) and a contiguous key range (a split of the prefix; the last
//     split also takes the tree block).  Each of its 8 waves (two per SIMD)
//     owns 32 query rows for the whole key range, so no merge between waves is
//     needed.  The query tile and 64-key K/V tiles are written into LDS by
//     direct global->LDS loads (XOR-swizzled rows; one K/V tile streams in
//     while the other is consumed); S^T = K Q^T and O^T += V^T P^T run on
//     v_mfma_f32_32x32x16_bf16, V^T fragments come straight from row-major V
//     through transposing LDS reads, and the online-softmax state is per lane
//     (each lane owns one query column).  A single split writes bf16 output
//     directly; several splits write partials (the normalised row O / l in
//     bf16, m and l in fp32) merged by k_attn_combine.
//  k_attn_valu<T>  generic fp32 / bf16 path, scalar FMA.
#include <float.h>
#include <math.h>

#include "sv_attn_dev.h"

namespace {

constexpr int AT_WAVES = 4;
constexpr int AT_THREADS = 64 * AT_WAVES;
constexpr int MF_WAVES = 8;                // waves of the MFMA kernel (two per SIMD)
constexpr int MF_THREADS = 64 * MF_WAVES;
constexpr int MF_QB = 1;                   // 32-row query blocks per wave
constexpr int KT = 64;  // keys per tile
#ifndef SV_ATTN_MIN_SPLIT_TILES
#define SV_ATTN_MIN_SPLIT_TILES 2  // a prefix split covers at least this many tiles
#endif
constexpr int TARGET_WG = 256;

struct AttnPlan {
  int32_t G, M, QB, QT, qtiles, nsplit, chunk, ntt, W, cap;
  float cscale;  // scale * log2(e)
  uint32_t pool_bytes;  // paged: bytes of one K (or V) pool, < 4 GiB
  uint16_t* opart;  // [units][nsplit][QT][D] bf16: the split's output row O / l
  float* mlpart;    // [units][nsplit][QT][2]: running max (scaled by log2 e) and l
};

// ------------------------------------------------------------------ MFMA path
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
  __device__ static __forceinline__ int swz(int r) {
    return CPR == 16 ? (((r << 1) & 14) | ((r >> 3) & 1)) : ((r & 6) | ((r >> 3) & 1));
  }
};

template <int D>
__global__ void __launch_bounds__(MF_THREADS, 2) k_attn_mfma(sv_attn_args a, AttnPlan p) {
  using TL = Tile<D>;
  constexpr int QB = MF_QB;             // 32-row query blocks per wave
  constexpr int KT64 = TL::KT;
  constexpr int DS = D / 16;            // 16-wide k-steps of S = K Q^T
  constexpr int DB = D / 32;            // 32-wide d-blocks of O^T
  constexpr uint32_t ROWB = TL::ROWB;
  // two tile buffers as separate arrays: the compiler can then tell that the loads
  // streaming into one never alias the reads of the other, and does not wait on them
  __shared__ __attribute__((aligned(1024))) unsigned char kvA[TL::BUF];
  __shared__ __attribute__((aligned(1024))) unsigned char kvB[TL::BUF];
  __shared__ __attribute__((aligned(1024))) unsigned char qsb[TL::QROWS * TL::ROWB];  // the work-group's query rows

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);  // uniform wave index
  const int lq = lane & 31;  // query column / key row inside a 32-block
  const int hf = lane >> 5;  // which half of the k dimension this lane feeds
  // the two waves sharing a SIMD get different issue priorities, so that one runs ahead
  // of the other inside each tile and its softmax overlaps the other's MFMAs
  if (w < MF_WAVES / 2) __builtin_amdgcn_s_setprio(1);

  // XCD-aware block order: consecutive logical ids land on the same XCD
  const int nb = gridDim.x;
  const int bid = blockIdx.x;
  const int lid = (nb % 8 == 0) ? (bid % 8) * (nb / 8) + bid / 8 : bid;
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
        int id = __builtin_amdgcn_readfirstlane(a.block_table[(int64_t)b * a.max_blocks + blk]);
        id = (id < 0 || id >= a.num_blocks) ? 0 : id;
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
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rK, (lds_void*)(kb + n * 1024), 16, off, soff, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rV, (lds_void*)(kb + TL::TBYTES + n * 1024), 16, off, soff, 0, 0);
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
    // the fragments of k-step ds + 1 are read while the MFMAs of step ds run, so the LDS
    // latency is hidden behind them
    sv_bf16x8 qf[2][QB], kf[2][2];
    auto frag = [&](int ds, int buf) {
      const int kslot = ((2 * ds + hf) ^ k_swz) * 16;  // Q and K rows share the swizzle of row lq
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        qf[buf][qb] = *(const sv_bf16x8*)(qsb + (w * 32 * QB + qb * 32) * ROWB + k_off + kslot);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) kf[buf][kb] = *(const sv_bf16x8*)(Kb + kb * 32 * ROWB + k_off + kslot);
    };
    frag(0, 0);
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      if (ds + 1 < DS) frag(ds + 1, (ds + 1) & 1);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          sacc[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ds & 1][kb], qf[ds & 1][qb], sacc[qb][kb], 0, 0, 0);
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
        uint64_t aw = qnode[qb] >= 0 ? a.anc_bits[((int64_t)b * N + qnode[qb]) * p.W + wi] : 0ull;
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
      float mt = sacc[qb][0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sacc[qb][kb][r]);
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      const float mnew = fmaxf(mrun[qb], mt);  // running maximum of the unscaled scores
      const float ms = mnew == -INFINITY ? 0.f : mnew * p.cscale;  // nothing visible yet: weights stay 0
      alpha[qb] = __builtin_amdgcn_exp2f(mrun[qb] * p.cscale - ms);
      moved |= mnew != mrun[qb];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          pf[qb][kb][r >> 3][r & 7] = (__bf16)__builtin_amdgcn_exp2f(fmaf(sacc[qb][kb][r], p.cscale, -ms));
      // the row sum of the bf16 weights the P V product uses: two per dot instruction
      float psum0 = 0.f, psum1 = 0.f;
      const sv_bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
          const sv_bf16x8 v = pf[qb][kb][t2];
          psum0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 0, 1), one2, psum0, false);
          psum1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 2, 3), one2, psum1, false);
          psum0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 4, 5), one2, psum0, false);
          psum1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 6, 7), one2, psum1, false);
        }
      float psum = psum0 + psum1;
      psum += __shfl_xor(psum, 32);
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
    // Half-steps of two d-blocks: the transposing reads of half-step h + 1 are issued before
    // the MFMAs of half-step h, which wait only for their own reads (LDS reads complete in
    // order, so at most the 4 newer reads may still be outstanding).
    constexpr int NH = 2 * DB;  // 4 steps (kb, t2) x DB / 2 halves
    uint2 vlo[2][2], vhi[2][2];
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
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      const int buf = h & 1;
      if (h + 1 < NH) {
        tr_issue(h + 1, buf ^ 1);
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
  if (!active) return;

  // ---- write: bf16 output (single split) or per-split partials: the normalised row
  // O / l in bf16 and (m, l) in fp32.  The wave stages its rows in its own query rows of
  // LDS (no other wave reads them, and its own reads of them are done), swizzled like the
  // query layout, then stores whole rows with 16 consecutive bytes per lane.
  const int unit = pair * p.qtiles + qtile;
  const int64_t pidx = (int64_t)unit * p.nsplit + split;
  unsigned char* ob = qsb + (w * 32 * QB) * ROWB;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int ql = w * 32 * QB + qb * 32 + lq;
    const int m = qtile * p.QT + ql;
    const float inv = lrun[qb] > 0.f ? 1.f / lrun[qb] : 0.f;
    if (p.nsplit > 1 && hf == 0 && m < p.M)
      *(float2*)(p.mlpart + (pidx * p.QT + ql) * 2) = make_float2(mrun[qb] * p.cscale, lrun[qb]);
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
      *(uint4*)(orow + ch * 8) = v;
    }
  }
}

// merge split partials: one wave per output row (b, node, head).  Every load
// of a row is issued before any is used (no data-dependent branch between
// them), so the merge costs one memory round trip, not one per split.
constexpr int AT_MAX_SPLIT_REG = 32;  // splits merged from registers (one round trip up to 32); more are streamed
template <int D>
__global__ void __launch_bounds__(256) k_attn_combine(sv_attn_args a, AttnPlan p) {
  const int lane = threadIdx.x & 63;
  const int64_t rowid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t nrows = (int64_t)a.B * a.N * a.Hq;
  if (rowid >= nrows) return;
  const int h = (int)(rowid % a.Hq);
  const int node = (int)((rowid / a.Hq) % a.N);
  const int b = (int)(rowid / ((int64_t)a.Hq * a.N));
  const int g = h / p.G;
  const int m = node * p.G + (h % p.G);
  const int qtile = m / p.QT, ql = m % p.QT;
  const int64_t unit = ((int64_t)b * a.Hkv + g) * p.qtiles + qtile;
  constexpr int EPL = D / 64;
  // lane s < nsplit holds split s's (m, l)
  const int ns = p.nsplit;
  float ms = -INFINITY, ls = 0.f;
  if (lane < ns) {
    const float2 ml = *(const float2*)(p.mlpart + ((unit * ns + lane) * p.QT + ql) * 2);
    ms = ml.x;
    ls = ml.y;
  }
  float mx = ms;
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  const float f = (ms == -INFINITY) ? 0.f : exp2f(ms - mx) * ls;  // weight of split `lane`'s normalised row
  float l = f;
  for (int o = 32; o > 0; o >>= 1) l += __shfl_xor(l, o);
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
  for (int s0 = 0; s0 < ns; s0 += AT_MAX_SPLIT_REG) {
    float part[AT_MAX_SPLIT_REG][EPL];
#pragma unroll
    for (int k = 0; k < AT_MAX_SPLIT_REG; ++k) {
      const int s = s0 + k;
      const uint16_t* orow = p.opart + ((unit * ns + (s < ns ? s : 0)) * p.QT + ql) * D + lane * EPL;
      if (EPL == 2) {
        const uint32_t two = *(const uint32_t*)orow;
        part[k][0] = s < ns ? __uint_as_float(two << 16) : 0.f;
        part[k][EPL - 1] = s < ns ? __uint_as_float(two & 0xffff0000u) : 0.f;
      } else {
#pragma unroll
        for (int e = 0; e < EPL; ++e) part[k][e] = s < ns ? bf16_bits_to_f32(orow[e]) : 0.f;
      }
    }
#pragma unroll
    for (int k = 0; k < AT_MAX_SPLIT_REG; ++k) {
      const float fk = __shfl(f, (s0 + k) & 63);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] += fk * part[k][e];
    }
  }
  const float inv = (mx != -INFINITY && l > 0.f) ? 1.f / l : 0.f;
  uint16_t* orow = (uint16_t*)a.out + rowid * D;
  if (EPL == 2) {
    *(uint32_t*)(orow + lane * 2) = f32_to_bf16_bits(acc[0] * inv) | ((uint32_t)f32_to_bf16_bits(acc[EPL - 1] * inv) << 16);
  } else {
#pragma unroll
    for (int e = 0; e < EPL; ++e) orow[lane * EPL + e] = f32_to_bf16_bits(acc[e] * inv);
  }
}

// ------------------------------------------------------------------ VALU path
// One work-group per (sequence, node, KV head); 256 keys per chunk, one key per
// thread for the scores; output (head, d) pairs strided over the threads.
template <typename T>
__global__ void __launch_bounds__(256) k_attn_valu(sv_attn_args a, AttnPlan p) {
  __shared__ float q_s[16 * 128];
  __shared__ float sc[16][256];
  __shared__ float o_s[16 * 128];
  __shared__ float m_s[16], l_s[16], al_s[16];
  __shared__ int64_t koff[256];
  __shared__ int ktree[256];
  const int t = threadIdx.x;
  const int id = blockIdx.x;
  const int g = id % a.Hkv;
  const int i = (id / a.Hkv) % a.N;
  const int b = id / (a.Hkv * a.N);
  const int G = p.G, D = a.D, N = a.N;
  if (a.status && i == 0 && g == 0) write_seq_status(a, b, p.cap);
  const T* qg = (const T*)a.q;
  const T* kc = (const T*)a.k_cache;
  const T* vc = (const T*)a.v_cache;
  const T* kt = (const T*)a.k_tree;
  const T* vt = (const T*)a.v_tree;
  for (int x = t; x < G * D; x += 256) {
    const int hh = x / D, d = x % D;
    q_s[x] = load_as_f32<T>(qg, (((int64_t)b * N + i) * a.Hq + g * G + hh) * D + d) * a.scale;
    o_s[x] = 0.f;
  }
  if (t < G) { m_s[t] = -INFINITY; l_s[t] = 0.f; }
  uint64_t anc[SV_MAX_W];
  for (int w = 0; w < SV_MAX_W; ++w) anc[w] = w < p.W ? a.anc_bits[((int64_t)b * N + i) * p.W + w] : 0ull;
  const int L = clamp_len(a.prefix_len[b], p.cap);
  const int total = L + N;
  __syncthreads();
  for (int c0 = 0; c0 < total; c0 += 256) {
    const int j = c0 + t;
    bool ok = false;
    int64_t off = 0;
    int istree = 0;
    if (j < L) {
      ok = true;
      if (a.paged) {
        int id2 = a.block_table[(int64_t)b * a.max_blocks + j / a.block_size];
        if (id2 < 0 || id2 >= a.num_blocks) id2 = 0;
        off = (((int64_t)id2 * a.Hkv + g) * a.block_size + j % a.block_size) * D;
      } else {
        off = (((int64_t)b * a.Hkv + g) * a.Lcap + j) * D;
      }
    } else if (j < total) {
      const int tt = j - L;
      const uint64_t wv = anc[tt >> 6];
      ok = (wv >> (tt & 63)) & 1ull;
      if (a.tree_in_cache) {  // node tt at cache position j = L + tt
        if (a.paged) {
          int id2 = a.block_table[(int64_t)b * a.max_blocks + j / a.block_size];
          if (id2 < 0 || id2 >= a.num_blocks) id2 = 0;
          off = (((int64_t)id2 * a.Hkv + g) * a.block_size + j % a.block_size) * D;
        } else {
          off = (((int64_t)b * a.Hkv + g) * a.Lcap + j) * D;
        }
      } else {
        off = (((int64_t)b * a.Hkv + g) * (N + 1) + tt + 1) * D;
        istree = 1;
      }
    }
    koff[t] = off;
    ktree[t] = ok ? istree : -1;
    const T* kb = istree ? kt : kc;
    for (int hh = 0; hh < G; ++hh) {
      float s = -INFINITY;
      if (ok) {
        s = 0.f;
        for (int d = 0; d < D; ++d) s = fmaf(q_s[hh * D + d], load_as_f32<T>(kb, off + d), s);
      }
      sc[hh][t] = s;
    }
    __syncthreads();
    // per-head online softmax update: wave w handles heads w, w+4, ...
    const int lane = t & 63, wv = t >> 6;
    for (int hh = wv; hh < G; hh += 4) {
      float mx = -INFINITY;
      for (int k = lane; k < 256; k += 64) mx = fmaxf(mx, sc[hh][k]);
      for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
      const float mold = m_s[hh];
      const float mnew = fmaxf(mold, mx);
      float sum = 0.f;
      for (int k = lane; k < 256; k += 64) {
        const float e = (mnew == -INFINITY || sc[hh][k] == -INFINITY) ? 0.f : expf(sc[hh][k] - mnew);
        sc[hh][k] = e;
        sum += e;
      }
      for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
      if (lane == 0) {
        const float al = (mold == -INFINITY) ? 0.f : expf(mold - mnew);
        al_s[hh] = (mnew == -INFINITY) ? 1.f : al;
        l_s[hh] = l_s[hh] * al_s[hh] + sum;
        m_s[hh] = mnew;
      }
    }
    __syncthreads();
    const int nk = min(256, total - c0);
    for (int x = t; x < G * D; x += 256) {
      const int hh = x / D, d = x % D;
      float acc = o_s[x] * al_s[hh];
      for (int k = 0; k < nk; ++k) {
        if (ktree[k] < 0) continue;
        const T* vb = ktree[k] ? vt : vc;
        acc = fmaf(sc[hh][k], load_as_f32<T>(vb, koff[k] + d), acc);
      }
      o_s[x] = acc;
    }
    __syncthreads();
  }
  for (int x = t; x < G * D; x += 256) {
    const int hh = x / D, d = x % D;
    const float v = l_s[hh] > 0.f ? o_s[x] / l_s[hh] : 0.f;
    const int64_t o = (((int64_t)b * N + i) * a.Hq + g * G + hh) * D + d;
    if (sizeof(T) == 4) ((float*)a.out)[o] = v;
    else ((uint16_t*)a.out)[o] = f32_to_bf16_bits(v);
  }
}

bool use_mfma(const sv_attn_args& a) {
  if (a.dtype != SV_BF16 || (a.D != 64 && a.D != 128)) return false;
  if (a.paged && (uint64_t)a.num_blocks * a.Hkv * a.block_size * a.D * 2 >= (1ull << 31)) return false;
  if (!a.paged && (uint64_t)a.Lcap * a.D * 2 >= (1ull << 31)) return false;
  if ((uint64_t)(a.N + 1) * a.D * 2 >= (1ull << 31)) return false;
  return true;
}

AttnPlan make_plan(const sv_attn_args& a) {
  AttnPlan p{};
  p.G = a.Hq / a.Hkv;
  p.M = a.N * p.G;
  p.W = (a.N + 63) / 64;
  // with the tree rows resident in the cache the prefix may fill only capacity - N positions
  p.cap = (a.paged ? a.max_blocks * a.block_size : a.Lcap) - (a.tree_in_cache ? a.N : 0);
  p.cscale = a.scale * LOG2E;
  p.pool_bytes = a.paged ? (uint32_t)((uint64_t)a.num_blocks * a.Hkv * a.block_size * a.D * 2) : 0u;
  if (!use_mfma(a)) {
    p.nsplit = 1;
    return p;
  }
  p.QB = MF_QB;
  p.QT = 32 * MF_QB * MF_WAVES;  // each wave owns 32 MF_QB query rows
  p.qtiles = (p.M + p.QT - 1) / p.QT;
  p.ntt = (a.N + KT - 1) / KT;
  const int64_t units = (int64_t)a.B * a.Hkv * p.qtiles;
  const int tiles_cap = (p.cap + KT - 1) / KT;
  int nsplit = (int)((TARGET_WG + units - 1) / units);
  const int max_split = tiles_cap / SV_ATTN_MIN_SPLIT_TILES > 1 ? tiles_cap / SV_ATTN_MIN_SPLIT_TILES : 1;
  if (nsplit > max_split) nsplit = max_split;
  if (nsplit > 64) nsplit = 64;  // the combine keeps one split per lane
  if (nsplit < 1) nsplit = 1;
  const int tiles_per = (tiles_cap + nsplit - 1) / nsplit;
  p.chunk = (tiles_per > 0 ? tiles_per : 1) * KT;
  p.nsplit = (p.cap + p.chunk - 1) / p.chunk;
  if (p.nsplit < 1) p.nsplit = 1;
  return p;
}

size_t workspace_bytes(const sv_attn_args& a, const AttnPlan& p) {
  if (!use_mfma(a) || p.nsplit == 1) return 0;
  const size_t units = (size_t)a.B * a.Hkv * p.qtiles;
  const size_t parts = units * p.nsplit * p.QT;
  const size_t obytes = (parts * a.D * sizeof(uint16_t) + 255) / 256 * 256;
  return obytes + parts * 2 * sizeof(float);
}

sv_status validate(const sv_attn_args& a) {
  if (a.B < 0 || a.N < 1 || a.N > SV_MAX_N || a.Hq < 1 || a.Hkv < 1 || a.Hq % a.Hkv) return SV_ERR_INVALID_ARGUMENT;
  if (a.Hq / a.Hkv > 16) return SV_ERR_UNSUPPORTED;
  if (a.D != 64 && a.D != 128) return SV_ERR_UNSUPPORTED;
  if (a.dtype != SV_F32 && a.dtype != SV_BF16) return SV_ERR_UNSUPPORTED;
  if (!(a.scale > 0.f) || !isfinite(a.scale)) return SV_ERR_INVALID_ARGUMENT;
  if (a.paged) {
    if (a.block_size != 16 || a.max_blocks < 1 || a.num_blocks < 1) return SV_ERR_INVALID_ARGUMENT;
  } else if (a.Lcap < 0) {
    return SV_ERR_INVALID_ARGUMENT;
  }
  if (a.tree_in_cache != 0 && a.tree_in_cache != 1) return SV_ERR_INVALID_ARGUMENT;
  if (a.tree_in_cache && (int64_t)(a.paged ? (int64_t)a.max_blocks * a.block_size : a.Lcap) < a.N)
    return SV_ERR_INVALID_ARGUMENT;
  return SV_OK;
}

}  // namespace

extern "C" size_t sv_tree_attention_workspace(const sv_attn_args* args) {
  if (!args || validate(*args) != SV_OK || args->B == 0) return 0;
  return workspace_bytes(*args, make_plan(*args));
}

extern "C" sv_status sv_tree_attention(const sv_attn_args* args, void* stream) {
  if (!args) return SV_ERR_INVALID_ARGUMENT;
  const sv_attn_args& a = *args;
  sv_status st = validate(a);
  if (st != SV_OK) return st;
  if (a.B == 0) return SV_OK;
  if (!a.q || !a.k_cache || !a.v_cache || (!a.tree_in_cache && (!a.k_tree || !a.v_tree)) || !a.prefix_len ||
      !a.anc_bits || !a.out)
    return SV_ERR_INVALID_ARGUMENT;
  if (a.paged && !a.block_table) return SV_ERR_INVALID_ARGUMENT;
  AttnPlan p = make_plan(a);
  const size_t need = workspace_bytes(a, p);
  if (need > 0) {
    if (!a.workspace || a.workspace_bytes < need || ((uintptr_t)a.workspace % 256)) return SV_ERR_INVALID_ARGUMENT;
    const size_t units = (size_t)a.B * a.Hkv * p.qtiles;
    const size_t parts = units * p.nsplit * p.QT;
    p.opart = (uint16_t*)a.workspace;
    p.mlpart = (float*)((char*)a.workspace + (parts * a.D * sizeof(uint16_t) + 255) / 256 * 256);
  }
  hipStream_t s = (hipStream_t)stream;
  if (use_mfma(a)) {
    const int64_t grid = (int64_t)a.B * a.Hkv * p.qtiles * p.nsplit;
    if (grid > 0x7fffffff) return SV_ERR_UNSUPPORTED;
    if (a.D == 128) hipLaunchKernelGGL(k_attn_mfma<128>, dim3(grid), dim3(MF_THREADS), 0, s, a, p);
    else hipLaunchKernelGGL(k_attn_mfma<64>, dim3(grid), dim3(MF_THREADS), 0, s, a, p);
    if (p.nsplit > 1) {
      const int64_t rows = (int64_t)a.B * a.N * a.Hq;
      const dim3 cg((unsigned)((rows + 3) / 4));
      if (a.D == 128) hipLaunchKernelGGL(k_attn_combine<128>, cg, dim3(256), 0, s, a, p);
      else hipLaunchKernelGGL(k_attn_combine<64>, cg, dim3(256), 0, s, a, p);
    }
  } else {
    const int64_t grid = (int64_t)a.B * a.N * a.Hkv;
    if (a.dtype == SV_F32) hipLaunchKernelGGL(k_attn_valu<float>, dim3(grid), dim3(256), 0, s, a, p);
    else hipLaunchKernelGGL(k_attn_valu<uint16_t>, dim3(grid), dim3(256), 0, s, a, p);
  }
  return sv_launch_status();
}
