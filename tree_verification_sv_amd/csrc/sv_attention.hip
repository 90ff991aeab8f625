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
//  k_attn_mfma<D, QB>  bf16, the hot path.  A work-group owns one KV head g of
//     one sequence, a tile of QT = 32*QB query rows (row m = node*G + head in
//     group, so the G query heads that share a KV head form one dense
//     contraction of M = N*G rows), and a contiguous key range (a split of the
//     prefix; the last split also takes the tree block).  Its 4 waves take
//     32-key tiles round-robin; each wave stages its tile through its own LDS
//     slice (K row-major, V transposed), computes S^T = K Q^T and O^T += V^T P^T
//     with v_mfma_f32_32x32x16_bf16, and keeps the online-softmax state per
//     lane (each lane owns one query column).  The 4 waves merge in LDS; a
//     single split writes bf16 output directly, several splits write fp32
//     partials (m, l, O) merged by k_attn_combine.
//  k_attn_valu<T>  generic fp32 / bf16 path (any D <= 128), scalar FMA.
#include <float.h>
#include <math.h>

#include "sv_common.h"

namespace {

constexpr int AT_WAVES = 4;
constexpr int AT_THREADS = 64 * AT_WAVES;
constexpr int KT = 32;  // keys per tile
constexpr float LOG2E = 1.4426950408889634f;
constexpr int TARGET_WG = 256;

struct AttnPlan {
  int32_t G, M, QB, QT, qtiles, nsplit, chunk, ntt, W, cap;
  float cscale;  // scale * log2(e)
  uint32_t pool_bytes;  // paged: bytes of one K (or V) pool, < 4 GiB
  float* opart;  // [units][nsplit][QT][D]
  float* mlpart; // [units][nsplit][QT][2]
};

__device__ __forceinline__ int clamp_len(int L, int cap) { return L < 0 ? 0 : (L > cap ? cap : L); }

// Data checks behind the optional status array, run by one work-group per
// sequence: 6 when prefix_len lies outside [0, capacity] (it is clamped), 5 when
// a needed block-table entry is the ghost block 0 or outside the pool (read as
// the ghost block).
__device__ void write_seq_status(const sv_attn_args& a, int b, int cap) {
  __shared__ int s_code;
  if (threadIdx.x == 0) s_code = 0;
  __syncthreads();
  const int L0 = a.prefix_len[b];
  if (L0 < 0 || L0 > cap) {
    if (threadIdx.x == 0) s_code = SV_SEQ_CAPACITY;
  } else if (a.paged) {
    const int nblk = (L0 + a.block_size - 1) / a.block_size;
    for (int k = threadIdx.x; k < nblk; k += blockDim.x) {
      const int id = a.block_table[(int64_t)b * a.max_blocks + k];
      if (id < 1 || id >= a.num_blocks) atomicOr(&s_code, SV_SEQ_BLOCK);
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) a.status[b] = s_code;
}

// ------------------------------------------------------------------ MFMA path
template <int D>
struct Lds {
  static constexpr int KSTR = D + 8;   // K row stride (bf16 elements), 16-byte padding
  static constexpr int VSTR = KT + 4;  // V^T row stride (bf16 elements), 8-byte padding
  static constexpr int K_ELEMS = KT * KSTR;
  static constexpr int V_ELEMS = D * VSTR;
  static constexpr int WAVE_ELEMS = K_ELEMS + V_ELEMS;
  static constexpr int STAGE_BYTES = AT_WAVES * WAVE_ELEMS * 2;
};

__device__ __forceinline__ uint32_t lo16(uint32_t x) { return x & 0xffffu; }
__device__ __forceinline__ uint32_t hi16(uint32_t x) { return x >> 16; }

// pack element e (0..7) of four 8-element bf16 vectors into 4 consecutive bf16
__device__ __forceinline__ uint2 pack_col(const uint4& a, const uint4& b, const uint4& c, const uint4& d, int e) {
  const int comp = e >> 1;
  const uint32_t xa = comp == 0 ? a.x : comp == 1 ? a.y : comp == 2 ? a.z : a.w;
  const uint32_t xb = comp == 0 ? b.x : comp == 1 ? b.y : comp == 2 ? b.z : b.w;
  const uint32_t xc = comp == 0 ? c.x : comp == 1 ? c.y : comp == 2 ? c.z : c.w;
  const uint32_t xd = comp == 0 ? d.x : comp == 1 ? d.y : comp == 2 ? d.z : d.w;
  if (e & 1) return make_uint2(hi16(xa) | (xb & 0xffff0000u), hi16(xc) | (xd & 0xffff0000u));
  return make_uint2(lo16(xa) | (xb << 16), lo16(xc) | (xd << 16));
}

template <int D, int QB>
__global__ void __launch_bounds__(AT_THREADS, 1) k_attn_mfma(sv_attn_args a, AttnPlan p) {
  using LD = Lds<D>;
  constexpr int DS = D / 16;                   // 16-wide k-steps of S = K Q^T
  constexpr int DB = D / 32;                   // 32-wide d-blocks of O^T
  constexpr int KPIECES = KT * (D / 8) / 64;   // 16-byte K pieces per lane per tile
  constexpr int VITEMS = (KT / 4) * (D / 8) / 64;  // (key quad, 8-d chunk) items per lane per tile
  constexpr int MERGE_BYTES = (2 * QB * DB * 16 * 64 + 2 * QB * 2 * 64) * 4;
  constexpr int SMEM_BYTES = LD::STAGE_BYTES > MERGE_BYTES ? LD::STAGE_BYTES : MERGE_BYTES;
  __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM_BYTES];

  const int lane = threadIdx.x & 63;
  // the wave index is uniform across the wave: keep tile bookkeeping in scalar registers
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lq = lane & 31;  // query column / row index inside a 32-block
  const int hf = lane >> 5;  // which half of the k dimension this lane feeds

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
  const int ntp = k1 > k0 ? (k1 - k0 + KT - 1) / KT : 0;
  const bool last = split == p.nsplit - 1;
  const int ntt = last ? p.ntt : 0;
  const int ntiles = ntp + ntt;

  const __bf16* qg = (const __bf16*)a.q;
  const uint16_t* kc = (const uint16_t*)a.k_cache;
  const uint16_t* vc = (const uint16_t*)a.v_cache;
  const uint16_t* kt = (const uint16_t*)a.k_tree;
  const uint16_t* vt = (const uint16_t*)a.v_tree;

  // ---- Q fragments (B operand of S^T = K Q^T): lane holds query column lq, d = 16*ds + 8*hf .. +7
  sv_bf16x8 qf[QB][DS];
  uint64_t anc[QB][SV_MAX_W];
  int qnode[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int m = qtile * p.QT + qb * 32 + lq;
    const bool valid = m < p.M;
    const int node = valid ? m / G : 0;
    const int h = g * G + (valid ? m % G : 0);
    qnode[qb] = node;
    const __bf16* qrow = qg + (((int64_t)b * N + node) * Hq + h) * D;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      if (valid) {
        qf[qb][ds] = *(const sv_bf16x8*)(qrow + ds * 16 + 8 * hf);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[qb][ds][e] = (__bf16)0.0f;
      }
    }
#pragma unroll
    for (int ww = 0; ww < SV_MAX_W; ++ww)
      anc[qb][ww] = (ntt > 0 && valid && ww < p.W) ? a.anc_bits[((int64_t)b * N + node) * p.W + ww] : 0ull;
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

  uint16_t* Ks = (uint16_t*)smem + w * LD::WAVE_ELEMS;
  uint16_t* VTs = Ks + LD::K_ELEMS;

  // ---- global -> register staging of one 32-key tile through buffer loads.
  // One buffer resource per source keeps the tile base in scalar registers;
  // lanes only add precomputed 32-bit offsets.  Keys past the valid range are
  // clamped onto the last valid key of the tile (finite data, masked out of
  // the softmax), so no load ever leaves the tensor.
  constexpr int CPR = D / 8;            // 16-byte chunks per row
  constexpr int QPI = 64 / CPR;         // V key-quads covered by one load instruction
  constexpr uint32_t ROWB = D * 2;      // bytes per K/V row
  const int64_t plane = (int64_t)b * a.Hkv + g;
  __amdgpu_buffer_rsrc_t rk, rv;
  const __amdgpu_buffer_rsrc_t rkt = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(kt + (plane * (N + 1) + 1) * D), 0, (int)(N * ROWB), 0x00020000);
  const __amdgpu_buffer_rsrc_t rvt = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(vt + (plane * (N + 1) + 1) * D), 0, (int)(N * ROWB), 0x00020000);
  if (a.paged) {
    rk = __builtin_amdgcn_make_buffer_rsrc((void*)kc, 0, (int)p.pool_bytes, 0x00020000);
    rv = __builtin_amdgcn_make_buffer_rsrc((void*)vc, 0, (int)p.pool_bytes, 0x00020000);
  } else {
    rk = __builtin_amdgcn_make_buffer_rsrc((void*)(kc + plane * a.Lcap * D), 0, (int)(a.Lcap * ROWB), 0x00020000);
    rv = __builtin_amdgcn_make_buffer_rsrc((void*)(vc + plane * a.Lcap * D), 0, (int)(a.Lcap * ROWB), 0x00020000);
  }
  // lane-constant key index and chunk of every load
  int kkey[KPIECES], kch[KPIECES];
#pragma unroll
  for (int it = 0; it < KPIECES; ++it) {
    kkey[it] = (lane + 64 * it) / CPR;
    kch[it] = (lane + 64 * it) % CPR;
  }
  const int vquad0 = lane % QPI, vch = lane / QPI;

  uint4 kreg[KPIECES];
  uint4 vreg[VITEMS][4];
  auto load_tile = [&](int tile) {
    const bool tree = tile >= ntp;
    // last valid key index inside this tile (wave-uniform)
    int klast;
    uint32_t offA = 0, offB = 0, soff = 0;
    if (tree) {
      const int t0 = (tile - ntp) * KT;
      klast = min(KT, N - t0) - 1;
      soff = (uint32_t)t0 * ROWB;
    } else {
      const int j0 = k0 + tile * KT;
      klast = min(KT, k1 - j0) - 1;
      if (a.paged) {
        // the tile spans two 16-token blocks; a block wholly past the end reuses the first
        int idA = a.block_table[(int64_t)b * a.max_blocks + j0 / 16];
        int idB = klast >= 16 ? a.block_table[(int64_t)b * a.max_blocks + j0 / 16 + 1] : idA;
        idA = (idA < 0 || idA >= a.num_blocks) ? 0 : idA;
        idB = (idB < 0 || idB >= a.num_blocks) ? 0 : idB;
        offA = (uint32_t)(((int64_t)idA * a.Hkv + g) * 16) * ROWB;
        offB = (uint32_t)(((int64_t)idB * a.Hkv + g) * 16) * ROWB;
      } else {
        soff = (uint32_t)j0 * ROWB;
      }
    }
    const bool paged_tile = !tree && a.paged;
    auto voffset = [&](int key, int ch) -> uint32_t {
      const int k = min(key, klast);
      if (paged_tile) return (k >= 16 ? offB : offA) + (uint32_t)(k & 15) * ROWB + ch * 16;
      return (uint32_t)k * ROWB + ch * 16;
    };
    const __amdgpu_buffer_rsrc_t rK = tree ? rkt : rk;
    const __amdgpu_buffer_rsrc_t rV = tree ? rvt : rv;
#pragma unroll
    for (int it = 0; it < KPIECES; ++it)
      kreg[it] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rK, voffset(kkey[it], kch[it]), soff, 0));
#pragma unroll
    for (int it = 0; it < VITEMS; ++it) {
      const int quad = vquad0 + QPI * it;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        vreg[it][kk] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rV, voffset(quad * 4 + kk, vch), soff, 0));
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int it = 0; it < KPIECES; ++it) *(uint4*)(Ks + kkey[it] * LD::KSTR + kch[it] * 8) = kreg[it];
#pragma unroll
    for (int it = 0; it < VITEMS; ++it) {
      const int quad = vquad0 + QPI * it;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        *(uint2*)(VTs + (vch * 8 + e) * LD::VSTR + quad * 4) =
            pack_col(vreg[it][0], vreg[it][1], vreg[it][2], vreg[it][3], e);
    }
  };

  int tile = w;
  if (tile < ntiles) load_tile(tile);
  for (; tile < ntiles; tile += AT_WAVES) {
    store_tile();
    const bool tree = tile >= ntp;
    const int j0 = k0 + tile * KT;
    const int t0 = (tile - ntp) * KT;
    const int nxt = tile + AT_WAVES;
    if (nxt < ntiles) load_tile(nxt);
    wave_lds_sync();

    // ---- S^T = K Q^T
    sv_f32x16 sacc[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[qb][r] = 0.f;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      const sv_bf16x8 kf = *(const sv_bf16x8*)(Ks + lq * LD::KSTR + ds * 16 + 8 * hf);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) sacc[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[qb][ds], sacc[qb], 0, 0, 0);
    }

    // ---- masks + online softmax (lane owns query column lq; keys 8*(r/4) + 4*hf + r%4)
    // Masks are needed only on the partial last prefix tile and on tree tiles;
    // both conditions are wave-uniform.
    const bool full = !tree && (j0 + KT <= k1);
    sv_bf16x8 pf[QB][2];
    bool moved = false;
    float alpha[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float s[16];
      if (full) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = sacc[qb][r] * p.cscale;
      } else if (!tree) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kk = 8 * (r >> 2) + 4 * hf + (r & 3);
          s[r] = (j0 + kk < k1) ? sacc[qb][r] * p.cscale : -INFINITY;
        }
      } else {
        const int wi = t0 >> 6;  // uniform: one 64-bit mask word covers the tile
        const uint64_t aw = wi == 0 ? anc[qb][0] : wi == 1 ? anc[qb][1] : wi == 2 ? anc[qb][2] : anc[qb][3];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int t = t0 + 8 * (r >> 2) + 4 * hf + (r & 3);
          const bool keep = (t < N) & (((aw >> (t & 63)) & 1ull) != 0);
          s[r] = keep ? sacc[qb][r] * p.cscale : -INFINITY;
        }
      }
      float mt = s[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mt = fmaxf(mt, s[r]);
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      const float mnew = fmaxf(mrun[qb], mt);
      const float msafe = mnew == -INFINITY ? 0.f : mnew;  // nothing visible yet: all weights stay 0
      alpha[qb] = __builtin_amdgcn_exp2f(mrun[qb] - msafe);
      moved |= mnew != mrun[qb];
      float psum = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = __builtin_amdgcn_exp2f(s[r] - msafe);
        psum += s[r];
      }
      psum += __shfl_xor(psum, 32);
      lrun[qb] = lrun[qb] * alpha[qb] + psum;
      mrun[qb] = mnew;
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int e = 0; e < 8; ++e) pf[qb][t2][e] = (__bf16)s[8 * t2 + e];
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

    // ---- O^T += V^T P^T
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const uint16_t* vrow = VTs + (db * 32 + lq) * LD::VSTR + 16 * t2 + 4 * hf;
        const uint2 lo = *(const uint2*)(vrow);
        const uint2 hi = *(const uint2*)(vrow + 8);
        uint4 raw = make_uint4(lo.x, lo.y, hi.x, hi.y);
        const sv_bf16x8 vf = *(const sv_bf16x8*)&raw;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          oacc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[qb][t2], oacc[qb][db], 0, 0, 0);
      }
    }
    wave_lds_sync();
  }

  // ---- merge the 4 waves: 2 -> 0, 3 -> 1, then 1 -> 0
  __syncthreads();
  float* mo = (float*)smem;                      // [2][QB][DB][16][64]
  float* mml = mo + 2 * QB * DB * 16 * 64;       // [2][QB][2][64]
  auto put = [&](int slot) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) mo[(((slot * QB + qb) * DB + db) * 16 + r) * 64 + lane] = oacc[qb][db][r];
      mml[((slot * QB + qb) * 2 + 0) * 64 + lane] = mrun[qb];
      mml[((slot * QB + qb) * 2 + 1) * 64 + lane] = lrun[qb];
    }
  };
  auto take = [&](int slot) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float mb = mml[((slot * QB + qb) * 2 + 0) * 64 + lane];
      const float lb = mml[((slot * QB + qb) * 2 + 1) * 64 + lane];
      const float m = fmaxf(mrun[qb], mb);
      if (m == -INFINITY) continue;
      const float fa = __builtin_amdgcn_exp2f(mrun[qb] - m), fb = __builtin_amdgcn_exp2f(mb - m);
      lrun[qb] = fa * lrun[qb] + fb * lb;
      mrun[qb] = m;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          oacc[qb][db][r] = fa * oacc[qb][db][r] + fb * mo[(((slot * QB + qb) * DB + db) * 16 + r) * 64 + lane];
    }
  };
  if (w >= 2) put(w - 2);
  __syncthreads();
  if (w < 2) take(w);
  __syncthreads();
  if (w == 1) put(0);
  __syncthreads();
  if (w != 0) return;
  take(0);

  // ---- write: bf16 output (single split) or fp32 partials
  const int unit = pair * p.qtiles + qtile;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int ql = qb * 32 + lq;
    const int m = qtile * p.QT + ql;
    if (m >= p.M) continue;
    if (p.nsplit == 1) {
      const float inv = lrun[qb] > 0.f ? 1.f / lrun[qb] : 0.f;
      const int node = qnode[qb];
      const int h = g * G + m % G;
      uint16_t* orow = (uint16_t*)a.out + (((int64_t)b * N + node) * Hq + h) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const int d = db * 32 + 8 * rq + 4 * hf;
          const uint32_t w0 = f32_to_bf16_bits(oacc[qb][db][4 * rq + 0] * inv) |
                              ((uint32_t)f32_to_bf16_bits(oacc[qb][db][4 * rq + 1] * inv) << 16);
          const uint32_t w1 = f32_to_bf16_bits(oacc[qb][db][4 * rq + 2] * inv) |
                              ((uint32_t)f32_to_bf16_bits(oacc[qb][db][4 * rq + 3] * inv) << 16);
          *(uint2*)(orow + d) = make_uint2(w0, w1);
        }
    } else {
      const int64_t pidx = (int64_t)unit * p.nsplit + split;
      float* orow = p.opart + (pidx * p.QT + ql) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const int d = db * 32 + 8 * rq + 4 * hf;
          *(float4*)(orow + d) = make_float4(oacc[qb][db][4 * rq + 0], oacc[qb][db][4 * rq + 1],
                                             oacc[qb][db][4 * rq + 2], oacc[qb][db][4 * rq + 3]);
        }
      if (hf == 0) {
        p.mlpart[(pidx * p.QT + ql) * 2 + 0] = mrun[qb];
        p.mlpart[(pidx * p.QT + ql) * 2 + 1] = lrun[qb];
      }
    }
  }
}

// merge split partials: one wave per output row (b, node, head).  Every load
// of a row is issued before any is used (no data-dependent branch between
// them), so the merge costs one memory round trip, not one per split.
constexpr int AT_MAX_SPLIT_REG = 16;  // splits merged from registers; more are streamed
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
  const float f = (ms == -INFINITY) ? 0.f : exp2f(ms - mx);  // weight of split `lane`
  float l = f * ls;
  for (int o = 32; o > 0; o >>= 1) l += __shfl_xor(l, o);
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
  for (int s0 = 0; s0 < ns; s0 += AT_MAX_SPLIT_REG) {
    float part[AT_MAX_SPLIT_REG][EPL];
#pragma unroll
    for (int k = 0; k < AT_MAX_SPLIT_REG; ++k) {
      const int s = s0 + k;
      const float* orow = p.opart + ((unit * ns + (s < ns ? s : 0)) * p.QT + ql) * D + lane * EPL;
#pragma unroll
      for (int e = 0; e < EPL; ++e) part[k][e] = s < ns ? orow[e] : 0.f;
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
      off = (((int64_t)b * a.Hkv + g) * (N + 1) + tt + 1) * D;
      istree = 1;
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
  p.cap = a.paged ? a.max_blocks * a.block_size : a.Lcap;
  p.cscale = a.scale * LOG2E;
  p.pool_bytes = a.paged ? (uint32_t)((uint64_t)a.num_blocks * a.Hkv * a.block_size * a.D * 2) : 0u;
  if (!use_mfma(a)) {
    p.nsplit = 1;
    return p;
  }
  p.QB = p.M <= 32 ? 1 : 2;
  p.QT = 32 * p.QB;
  p.qtiles = (p.M + p.QT - 1) / p.QT;
  p.ntt = (a.N + KT - 1) / KT;
  const int64_t units = (int64_t)a.B * a.Hkv * p.qtiles;
  const int tiles_cap = (p.cap + KT - 1) / KT;
  int nsplit = (int)((TARGET_WG + units - 1) / units);
  const int max_split = tiles_cap / AT_WAVES > 1 ? tiles_cap / AT_WAVES : 1;
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
  const size_t obytes = (parts * a.D * sizeof(float) + 255) / 256 * 256;
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
  if (!a.q || !a.k_cache || !a.v_cache || !a.k_tree || !a.v_tree || !a.prefix_len || !a.anc_bits || !a.out)
    return SV_ERR_INVALID_ARGUMENT;
  if (a.paged && !a.block_table) return SV_ERR_INVALID_ARGUMENT;
  AttnPlan p = make_plan(a);
  const size_t need = workspace_bytes(a, p);
  if (need > 0) {
    if (!a.workspace || a.workspace_bytes < need || ((uintptr_t)a.workspace % 256)) return SV_ERR_INVALID_ARGUMENT;
    const size_t units = (size_t)a.B * a.Hkv * p.qtiles;
    const size_t parts = units * p.nsplit * p.QT;
    p.opart = (float*)a.workspace;
    p.mlpart = (float*)((char*)a.workspace + (parts * a.D * sizeof(float) + 255) / 256 * 256);
  }
  hipStream_t s = (hipStream_t)stream;
  if (use_mfma(a)) {
    const int64_t grid = (int64_t)a.B * a.Hkv * p.qtiles * p.nsplit;
    if (grid > 0x7fffffff) return SV_ERR_UNSUPPORTED;
    if (a.D == 128) {
      if (p.QB == 1) hipLaunchKernelGGL((k_attn_mfma<128, 1>), dim3(grid), dim3(AT_THREADS), 0, s, a, p);
      else hipLaunchKernelGGL((k_attn_mfma<128, 2>), dim3(grid), dim3(AT_THREADS), 0, s, a, p);
    } else {
      if (p.QB == 1) hipLaunchKernelGGL((k_attn_mfma<64, 1>), dim3(grid), dim3(AT_THREADS), 0, s, a, p);
      else hipLaunchKernelGGL((k_attn_mfma<64, 2>), dim3(grid), dim3(AT_THREADS), 0, s, a, p);
    }
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
