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

#ifndef SV_ATTN_MIN_SPLIT_TILES
#define SV_ATTN_MIN_SPLIT_TILES 2  // a prefix split covers at least this many tiles
#endif
constexpr int TARGET_WG = 256;
constexpr int AT_WAVES = 4;
constexpr int AT_THREADS = 64 * AT_WAVES;
// ------------------------------------------------------------------ MFMA path
// Batches whose work-groups each own a whole (sequence, KV head) pair -- one query tile, one
// split -- are dispatched longest sequence first: with prefix lengths of very different sizes
// (a batch of live requests) an in-order dispatch leaves the last long sequences running alone
// on a few CUs, while longest-first list scheduling bounds the tail by the shortest jobs.  A
// batch whose lengths are all equal keeps the XCD-aware order (measured faster there).
constexpr int AT_LPT_MAX_B = 256;  // batches up to this size are ordered (one LDS scan of B lengths)

bool attn_longest_first(const sv_attn_args& a, const AttnPlan& p) {
  return p.nsplit == 1 && p.qtiles == 1 && a.B > 1 && a.B <= AT_LPT_MAX_B;
}

template <int D>
__global__ void __launch_bounds__(MF_THREADS, 2) k_attn_mfma(sv_attn_args a, AttnPlan p, int longest_first) {
  __shared__ __attribute__((aligned(1024))) unsigned char kvA[Tile<D>::BUF];
  __shared__ __attribute__((aligned(1024))) unsigned char kvB[Tile<D>::BUF];
  __shared__ __attribute__((aligned(1024))) unsigned char qsb[Tile<D>::QROWS * Tile<D>::ROWB];
  __shared__ int32_t s_bt[AT_BT_MAX];
  const int nb = gridDim.x;
  const int bid = blockIdx.x;
  int lid = -1;
  if (longest_first) {  // uniform
    // block bid takes the pair (sequence of rank bid / Hkv by length, KV head bid % Hkv): the
    // round-robin placement of blocks on XCDs then gives every XCD the same mix of lengths, and
    // each XCD starts its longest work first.  Rank: longer first, lower index first on ties.
    const int r = bid / a.Hkv, t = threadIdx.x, lane = t & 63, w = t >> 6;
    __shared__ int32_t s_pick;
    for (int i = t; i < a.B; i += MF_THREADS) s_bt[i] = clamp_len(a.prefix_len[i], p.cap);
    __syncthreads();
    // every wave holds all B lengths (lane j % 64 of register j / 64; -1 past B) and ranks
    // i = w, w + 8, ... with one ballot per 64 lengths; lane k holds the length of its k-th i
    constexpr int NQ = AT_LPT_MAX_B / 64;
    int lj[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) lj[q] = 64 * q + lane < a.B ? s_bt[64 * q + lane] : -1;
    const int l0 = s_bt[0];
    uint64_t differ = 0;
#pragma unroll
    for (int q = 0; q < NQ; ++q) differ |= __ballot(lj[q] >= 0 && lj[q] != l0);
    if (!differ) s_pick = -1;  // equal lengths (every wave sees the same): the XCD-aware order below
    const int mine = w + MF_WAVES * lane;
    const int lmine = mine < a.B ? s_bt[mine] : 0;
    for (int k = 0; differ && w + MF_WAVES * k < a.B; ++k) {  // uniform per wave
      const int i = w + MF_WAVES * k;
      const int li = __shfl(lmine, k);
      int rank = 0;
#pragma unroll
      for (int q = 0; q < NQ; ++q)
        rank += __popcll(__ballot((lj[q] > li) | ((lj[q] == li) & (64 * q + lane < i))));
      if (rank == r && lane == 0) s_pick = i;  // ranks are a permutation of 0 .. B-1: one writer
    }
    __syncthreads();
    const int pick = s_pick;
    lid = pick >= 0 ? pick * a.Hkv + bid % a.Hkv : -1;
    __syncthreads();  // s_bt is the block-id table of the body from here on
  }
  // XCD-aware block order: consecutive logical ids land on the same XCD
  if (!longest_first || lid < 0) lid = (nb % 8 == 0) ? (bid % 8) * (nb / 8) + bid / 8 : bid;
  attn_mfma_body<D>(a, p, lid, kvA, kvB, qsb, nullptr, 0, nullptr, s_bt);
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

}  // namespace

// Argument checks of sv_tree_attention (also used by the one-launch step).
sv_status sv_attn_validate(const sv_attn_args& a) {
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

namespace {

}  // namespace

extern "C" size_t sv_tree_attention_workspace(const sv_attn_args* args) {
  if (!args || sv_attn_validate(*args) != SV_OK || args->B == 0) return 0;
  return workspace_bytes(*args, make_plan(*args));
}

extern "C" sv_status sv_tree_attention(const sv_attn_args* args, void* stream) {
  if (!args) return SV_ERR_INVALID_ARGUMENT;
  const sv_attn_args& a = *args;
  sv_status st = sv_attn_validate(a);
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
    const int lf = attn_longest_first(a, p) ? 1 : 0;
    if (a.D == 128) hipLaunchKernelGGL(k_attn_mfma<128>, dim3(grid), dim3(MF_THREADS), 0, s, a, p, lf);
    else hipLaunchKernelGGL(k_attn_mfma<64>, dim3(grid), dim3(MF_THREADS), 0, s, a, p, lf);
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
