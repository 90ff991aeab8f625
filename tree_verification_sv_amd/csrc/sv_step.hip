// The whole verification step in one launch: tree tensorisation, ancestor-masked
// tree attention, speculative acceptance with the bonus token, and the commit of
// the accepted path.
//
// "EAGLE-Pangu: Accelerator-Safe Tree Speculative Decoding on Ascend NPUs",
// technical summary sec. 2 ("Ejecucion del Maestro con Mascara de Arbol
// Fusionada": the tree mask is built inside the target's execution instead of as
// a separate pass) and sec. 4 (mask construction and tensorisation overhead,
// with verification and cache commit dominating the step).  "Accelerating Sonar
// Through Speculation", section "Inferencia con Decodificacion Especulativa":
// the accepted count stays on the device.
//
// A step of the separate calls is a chain of dependent launches whose gaps,
// not bytes, set its time at batch 1.  Here one grid runs four regions of
// 512-thread work-groups, one per compute unit, in dispatch order (each region
// starts on a multiple of 8 blocks, so its blocks keep the round-robin XCD
// order):
//   1. attention work-groups (the MFMA attention body of sv_attn_dev.h, eight
//      waves, two per SIMD): the longest chain of the step, so they take their
//      compute units first; the last split of each (sequence, KV head) pair
//      derives its query nodes' ancestor sets from the parent array itself;
//   2. the mask outputs, when the caller asks for them (one work-group per
//      sequence; nothing else reads them);
//   3. acceptance groups, one per row (over wide trees the stochastic and top-K
//      walks resolve only rows with a usable child and the root: a walk that
//      stops at a leaf draws that row's bonus in the walker's work-group);
//   4. merge work-groups, which wait for the attention splits they combine --
//      only for work-groups dispatched before them, so the wait always ends.
// The roles share the LDS (a work-group runs one role): the attention's tile and query
// buffers, and one union of the other roles' state.
#include "sv_accept_dev.h"
#include "sv_attn_dev.h"

namespace {

constexpr int SS_TARGET_WG = 96;    // attention work-groups aimed at (the acceptance takes most compute units)
constexpr int SS_MIN_TILES = 2;     // 64-key tiles per split at least

struct StepKArgs {
  sv_attn_args at;
  AttnPlan ap;
  sv_accept_args ac;
  AccWs ws;
  sv_commit_args cm;
  int32_t has_cm, G;
  uint64_t* m_anc;      // mask outputs (nullable)
  int32_t* m_depth;
  int32_t* m_path;
  int32_t* m_status;
  int32_t r_mask, r_acc, r_merge, r_end;  // first block of regions 2..4, and the grid size
  int32_t nacc;         // acceptance work-groups
  uint32_t* exit_count; // work-groups of the launch that have finished
};

template <typename T, int TH, bool STO>
union StepAux {  // the fourth LDS array: acceptance state, or the attention's / merge's / mask's scratch
  AccShared<T, TH, STO> acc;
  struct {
    uint64_t anc[SV_MAX_N * 4];
    int32_t spar[SV_MAX_N];
  } att;
  float mrg[TH / 8 * 64];
  struct {
    int32_t spar[SV_MAX_N];
    int32_t worst;
  } mask;
};

template <int D, int MODE>
__global__ void __launch_bounds__(MF_THREADS, 1) k_verify_step(StepKArgs k) {
  constexpr bool STO = MODE != SV_GREEDY;
  constexpr int TH = MF_THREADS;
  using T = uint16_t;
  using TL = Tile<D>;
  __shared__ __attribute__((aligned(1024))) unsigned char s_kvA[TL::BUF];
  __shared__ __attribute__((aligned(1024))) unsigned char s_kvB[TL::BUF];
  __shared__ __attribute__((aligned(1024))) unsigned char s_q[TL::QROWS * TL::ROWB];
  __shared__ StepAux<T, TH, STO> s_aux;
  const int bid = blockIdx.x;
  if (bid < k.r_mask) {
    // ---- attention: XCD-aware order (consecutive logical ids on one XCD)
    const int nb = k.r_mask;
    const int lid = (bid % 8) * (nb / 8) + bid / 8;
    if (lid < k.ap.nwg)
      attn_mfma_body<D>(k.at, k.ap, lid, s_kvA, s_kvB, s_q, k.ac.parents, k.ac.max_depth, (unsigned char*)&s_aux);
  } else if (bid < k.r_acc) {
    // ---- mask outputs, one work-group per sequence
    const int b = bid - k.r_mask;
    if (b < k.ac.B)
      mask_seq(k.ac.parents, k.ac.N, k.ac.max_depth, (k.ac.N + 63) / 64, k.m_anc, k.m_depth, k.m_path, k.m_status, b,
               s_aux.mask.spar, &s_aux.mask.worst);
  } else if (bid < k.r_merge) {
    // ---- acceptance
    const AccRole role{bid - k.r_acc, k.nacc, (k.ac.N + 1) * k.G};
    accept_body<T, MODE, true, TH, false, false>(k.ac, k.G, k.ws, k.cm, k.has_cm, role, s_aux.acc);
  } else {
    // ---- merge of the attention splits
    const int pos = bid - k.r_merge, nb = k.r_end - k.r_merge;
    const int mid = (pos % 8) * (nb / 8) + pos / 8;
    if (mid < k.ac.B * k.at.Hkv * k.ap.mper) step_merge<D, TH>(k.at, k.ap, mid, s_aux.mrg);
  }
  // ---- the last work-group of the launch leaves the attention's arrival counters zeroed.  The
  // merge work-groups read those counters before they count out (their polls have returned), so
  // once every work-group has counted out no read of them is left.
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t o = __hip_atomic_fetch_add(k.exit_count, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (o + 1 == gridDim.x) {
      for (int u = 0; u < k.ap.nunits && k.ap.nsplit > 1; ++u)
        __hip_atomic_store(&k.ap.arrive[u], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(k.exit_count, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

bool attn_fits(const sv_attn_args& a) {
  if (a.dtype != SV_BF16 || (a.D != 64 && a.D != 128)) return false;
  if (a.paged && (uint64_t)a.num_blocks * a.Hkv * a.block_size * a.D * 2 >= (1ull << 31)) return false;
  if (!a.paged && (uint64_t)a.Lcap * a.D * 2 >= (1ull << 31)) return false;
  if ((uint64_t)(a.N + 1) * a.D * 2 >= (1ull << 31)) return false;
  return true;
}

AttnPlan step_plan(const sv_attn_args& a) {
  AttnPlan p{};
  p.G = a.Hq / a.Hkv;
  p.M = a.N * p.G;
  p.W = (a.N + 63) / 64;
  p.cap = (a.paged ? a.max_blocks * a.block_size : a.Lcap) - (a.tree_in_cache ? a.N : 0);
  p.cscale = a.scale * LOG2E;
  p.pool_bytes = a.paged ? (uint32_t)((uint64_t)a.num_blocks * a.Hkv * a.block_size * a.D * 2) : 0u;
  p.QB = MF_QB;
  p.QT = 32 * MF_QB * MF_WAVES;
  p.qtiles = (p.M + p.QT - 1) / p.QT;
  p.ntt = (a.N + KT - 1) / KT;
  p.nunits = a.B * a.Hkv * p.qtiles;
  const int tiles_cap = (p.cap + KT - 1) / KT;
  int nsplit = (SS_TARGET_WG + p.nunits - 1) / p.nunits;
  const int max_split = tiles_cap / SS_MIN_TILES > 1 ? tiles_cap / SS_MIN_TILES : 1;
  if (nsplit > max_split) nsplit = max_split;
  if (nsplit > 64) nsplit = 64;  // the merge keeps one weight per split and row
  if (nsplit < 1) nsplit = 1;
  const int tiles_per = (tiles_cap + nsplit - 1) / nsplit;
  p.chunk = (tiles_per > 0 ? tiles_per : 1) * KT;
  p.nsplit = (p.cap + p.chunk - 1) / p.chunk;
  if (p.nsplit < 1) p.nsplit = 1;
  p.nwg = p.nunits * p.nsplit;
  p.mrows = MF_THREADS / (a.D / 8);  // one pass of a merge work-group
  p.mper = p.nsplit > 1 ? (p.M + p.mrows - 1) / p.mrows : 0;
  return p;
}

int step_G(const sv_accept_args& a) { return launch_G(a, MF_THREADS); }

struct StepLayout {
  WsLayout acc;
  size_t opart, mlpart, arrive, exitc, total;
};
StepLayout step_layout(const sv_attn_args& at, const sv_accept_args& ac, const AttnPlan& p) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  StepLayout l{};
  l.acc = ws_layout_g(ac, step_G(ac), 1);
  size_t o = l.acc.total;
  const size_t parts = (size_t)p.nunits * (p.nsplit > 1 ? p.nsplit : 0) * p.QT;
  l.opart = o; o = up(o + parts * at.D * sizeof(uint16_t));
  l.mlpart = o; o = up(o + parts * 2 * sizeof(float));
  l.arrive = o; o = up(o + (size_t)p.nunits * sizeof(uint32_t));
  l.exitc = o; o = up(o + sizeof(uint32_t));
  l.total = o;
  return l;
}

sv_status step_check(const sv_step_args& s) {
  if (!s.attn || !s.accept) return SV_ERR_INVALID_ARGUMENT;
  const sv_attn_args& at = *s.attn;
  const sv_accept_args& ac = *s.accept;
  sv_status st = sv_attn_validate(at);
  if (st != SV_OK) return st;
  if (ac.B != at.B || ac.N != at.N || ac.N < 1 || ac.N > SV_MAX_N || ac.V < 1 || ac.max_depth < 1 ||
      ac.max_depth > SV_MAX_DEPTH)
    return SV_ERR_INVALID_ARGUMENT;
  if (ac.mode != SV_GREEDY && ac.mode != SV_STOCHASTIC && ac.mode != SV_TOPK_DRAFT) return SV_ERR_UNSUPPORTED;
  if (ac.flags != 0) return SV_ERR_UNSUPPORTED;
  if (!attn_fits(at) || ac.logits_dtype != SV_BF16) return SV_ERR_UNSUPPORTED;
  // logits rows on 16 bytes (whole 16-byte pieces of a row)
  if ((ac.V % 8) != 0 || ((uintptr_t)ac.target_logits % 16) != 0 ||
      (ac.mode == SV_STOCHASTIC && ((uintptr_t)ac.draft_logits % 16) != 0))
    return SV_ERR_UNSUPPORTED;
  if (step_G(ac) > AC_MAXG) return SV_ERR_UNSUPPORTED;
  if (at.tree_in_cache && ac.commit) return SV_ERR_UNSUPPORTED;  // the commit would move rows the attention reads
  const bool mo = s.anc_bits || s.depth || s.mask_status || s.path_rows;
  if (mo && (!s.anc_bits || !s.depth || !s.mask_status)) return SV_ERR_INVALID_ARGUMENT;
  return SV_OK;
}

}  // namespace

extern "C" size_t sv_verify_step_workspace(const sv_step_args* s) {
  if (!s || step_check(*s) != SV_OK || s->attn->B == 0) return 0;
  return step_layout(*s->attn, *s->accept, step_plan(*s->attn)).total;
}

extern "C" sv_status sv_verify_step(const sv_step_args* sp, void* stream) {
  if (!sp) return SV_ERR_INVALID_ARGUMENT;
  const sv_step_args& s = *sp;
  sv_status st = step_check(s);
  if (st != SV_OK) return st;
  const sv_attn_args& at = *s.attn;
  const sv_accept_args& ac = *s.accept;
  if (at.B == 0) return SV_OK;
  if (!at.q || !at.k_cache || !at.v_cache || (!at.tree_in_cache && (!at.k_tree || !at.v_tree)) || !at.prefix_len ||
      !at.out || (at.paged && !at.block_table))
    return SV_ERR_INVALID_ARGUMENT;
  if (!ac.parents || !ac.tokens || !ac.target_logits || !ac.accept_len || !ac.accept_rows || !ac.out_tokens ||
      !ac.num_out || !ac.stop_row || !ac.status)
    return SV_ERR_INVALID_ARGUMENT;
  if (ac.mode == SV_STOCHASTIC && !ac.draft_logits) return SV_ERR_INVALID_ARGUMENT;
  if (ac.mode != SV_GREEDY && (!ac.u_accept || !ac.u_sample || !(ac.temperature > 0.f))) return SV_ERR_INVALID_ARGUMENT;
  const AttnPlan p0 = step_plan(at);
  const StepLayout l = step_layout(at, ac, p0);
  if (!s.workspace || s.workspace_bytes < l.total || ((uintptr_t)s.workspace % 256)) return SV_ERR_INVALID_ARGUMENT;
  StepKArgs k{};
  k.at = at;
  k.at.anc_bits = nullptr;  // derived in the launch
  k.ap = p0;
  char* base = (char*)s.workspace;
  k.ap.opart = (uint16_t*)(base + l.opart);
  k.ap.mlpart = (float*)(base + l.mlpart);
  k.ap.arrive = (uint32_t*)(base + l.arrive);
  k.exit_count = (uint32_t*)(base + l.exitc);
  k.ac = ac;
  k.ac.anc_bits = nullptr;  // depths and root paths come from the parents
  k.ac.depth = nullptr;
  k.ac.workspace = s.workspace;
  k.ac.workspace_bytes = l.acc.total;
  k.ws = ws_views(s.workspace, l.acc);
  if (ac.commit) {
    st = svc::walker_commit_ok(*ac.commit, ac.B, ac.N, ac.max_depth);
    if (st != SV_OK) return st;
    k.cm = *ac.commit;
    k.has_cm = 1;
  }
  k.G = step_G(ac);
  k.m_anc = s.anc_bits;
  k.m_depth = s.depth;
  k.m_path = s.path_rows;
  k.m_status = s.mask_status;
  auto up8 = [](int64_t x) { return (x + 7) / 8 * 8; };
  const int64_t nacc = num_groups(ac) * k.G;  // a multiple of 8 * G
  const int64_t nmask = s.anc_bits ? up8(ac.B) : 0;
  const int64_t natt = up8(p0.nwg);
  const int64_t nmerge = up8((int64_t)ac.B * at.Hkv * p0.mper);
  const int64_t total = natt + nmask + nacc + nmerge;
  if (total > 0x7fffffff) return SV_ERR_UNSUPPORTED;
  k.r_mask = (int32_t)natt;
  k.r_acc = (int32_t)(natt + nmask);
  k.r_merge = (int32_t)(k.r_acc + nacc);
  k.r_end = (int32_t)total;
  k.nacc = (int32_t)nacc;
  hipStream_t hs = (hipStream_t)stream;
  const dim3 grid((unsigned)total), block(MF_THREADS);
#define SV_STEP(D_, M_) hipLaunchKernelGGL((k_verify_step<D_, M_>), grid, block, 0, hs, k)
  if (at.D == 128) {
    if (ac.mode == SV_STOCHASTIC) SV_STEP(128, SV_STOCHASTIC);
    else if (ac.mode == SV_TOPK_DRAFT) SV_STEP(128, SV_TOPK_DRAFT);
    else SV_STEP(128, SV_GREEDY);
  } else {
    if (ac.mode == SV_STOCHASTIC) SV_STEP(64, SV_STOCHASTIC);
    else if (ac.mode == SV_TOPK_DRAFT) SV_STEP(64, SV_TOPK_DRAFT);
    else SV_STEP(64, SV_GREEDY);
  }
#undef SV_STEP
  return sv_launch_status();
}
