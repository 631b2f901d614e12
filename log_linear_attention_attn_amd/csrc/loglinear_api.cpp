// C ABI of the log-linear attention library: argument validation (host only,
// before any HIP call), planning of the segmented sweep, workspace handling
// and kernel dispatch.  Semantics of every entry point: include/loglinear.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <initializer_list>
#include <mutex>

#include "ll_internal.h"
#include "loglinear.h"

namespace {

int bit_length(long long x) {
  int n = 0;
  while (x > 0) {
    ++n;
    x >>= 1;
  }
  return n;
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

struct FwdPlan {
  int BH, N, L, DKP, seg_log2, nseg, nslot;
  int blk_log2, nblk1;  // state blocks: 2^blk_log2 chunks; slots per (b,h)
  size_t ws_state, ws_nodes, ws_decay, ws_bdecay, ws_total;
};

// Chunks per segment.  The register-state sweep runs one 512-thread workgroup
// per CU (its LDS use), each walking its segment's chunks in order, so the
// critical path is (rounds of workgroups over the 256 CUs of an MI355X) x
// (chunks per segment + ~2 chunks' worth of prologue): the segment size
// minimising that, the largest on a tie (fewer segment states, less prologue
// traffic, one round instead of several), up to 1024 chunks.  Other
// shapes (16 dv columns per workgroup, several workgroups per CU): the largest
// size, up to 16 chunks, that still gives at least 2048 workgroups.  Depends
// on shapes only, so the workspace size is known without the dtype.
constexpr long long kCUs = 256;
// Whether the automatic choice takes the full-width sweep for the shapes it
// covers (it needs 8 segments per (b,h) at B=2 H=16 T=16384, whose segment
// prepass costs more than its faster sweep saves, so not yet).
constexpr bool kWideAuto = false;

// The kernels move q, k, v, out and the level states with 16-byte vector
// accesses; pointers that are not 16-byte aligned are rejected up front.
bool aligned16(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (reinterpret_cast<uintptr_t>(p) & 15) return false;
  return true;
}

int auto_seg_log2(long long BH, int dk, int dv, int C, int N, int L) {
  const int nslot = N > 1 ? bit_length(N - 1) : 0;
  const bool wide_shape = kWideAuto && ll::sweep_wide_ok(C, dk, dv, L, nslot, -1);
  const bool rs_shape = C == 64 && dk > 64 && dv % 64 == 0 && N <= 1024;
  if (wide_shape) {
    // full-width sweep: one workgroup (all 128 columns) per (b,h, segment),
    // one per CU; among the segment sizes it is built for, the one that
    // minimises rounds x (chunks per segment + ~2 chunks of prologue), the
    // largest on a tie
    int best = -1;
    long long best_cost = -1;
    for (int s = 6; s >= 3; --s) {
      if (!ll::sweep_wide_seg_ok(s, nslot)) continue;
      const long long nseg = (N + (1LL << s) - 1) >> s;
      const long long rounds = (BH * nseg + kCUs - 1) / kCUs;
      const long long cost = rounds * (std::min<long long>(1LL << s, N) + 2);
      if (best_cost < 0 || cost < best_cost) {
        best_cost = cost;
        best = s;
      }
    }
    if (best >= 0) return best;
  }
  if (rs_shape) {
    // workgroups per segment: one per 64 columns
    const long long per_seg = BH * (dv / 64);
    int best = 6;
    long long best_cost = -1;
    for (int s = 10; s >= 0; --s) {
      const long long nseg = (N + (1LL << s) - 1) >> s;
      const long long rounds = (per_seg * nseg + kCUs - 1) / kCUs;
      const long long cost = rounds * (std::min<long long>(1LL << s, N) + 2);
      if (best_cost < 0 || cost < best_cost) {
        best_cost = cost;
        best = s;
      }
    }
    return best;
  }
  const long long per_seg = BH * (dv / 16);
  int s = 4;
  while (s > 0) {
    const long long nseg = (N + (1LL << s) - 1) >> s;
    if (per_seg * nseg >= 2048) break;
    --s;
  }
  return s;
}

// Chunks per state block: segments are split into blocks until the state
// kernel has at least 512 workgroups (one per (b,h, block, 64 dv columns)),
// keeping at least 8 chunks per block; the node kernel adds the blocks up.
int auto_blk_log2(long long BH, int dv, int seg_log2, int nseg) {
  const long long per = BH * (nseg - 1) * (dv >= 64 ? dv / 64 : 1);
  int b = seg_log2;
  while (b > 3 && (per << (seg_log2 - b)) < 512) --b;
  return b;
}

// Heads per q/k head for qk_heads q/k heads (0 = one per head); 0 if
// qk_heads does not divide H.
int heads_per_qk(int H, int qk_heads) {
  if (qk_heads == 0 || qk_heads == H) return 1;
  if (qk_heads < 0 || H <= 0 || H % qk_heads != 0) return 0;
  return H / qk_heads;
}

int plan_fwd(int B, int H, int T, int dk, int dv, int C, int seg_log2, FwdPlan* p) {
  if (B < 0 || H < 0 || T < 0) return LL_ERR_SHAPE;
  if (C <= 0 || (C & (C - 1)) != 0) return LL_ERR_SHAPE;
  if (C != 16 && C != 32 && C != 64) return LL_ERR_UNSUPPORTED;
  if (dk < 16 || dk % 16 != 0 || dv < 16 || dv % 16 != 0) return LL_ERR_SHAPE;
  if (dk > 128 || dv > 1024) return LL_ERR_UNSUPPORTED;
  if (T > (1 << 28)) return LL_ERR_UNSUPPORTED;
  if (seg_log2 < -1 || seg_log2 > 12) return LL_ERR_SHAPE;
  if ((long long)B * H > (1LL << 24)) return LL_ERR_UNSUPPORTED;
  p->BH = B * H;
  p->N = T > 0 ? (T + C - 1) / C : 0;
  p->L = T > 0 ? bit_length(T - 1) + 1 : 0;
  p->DKP = dk <= 32 ? 32 : (dk <= 64 ? 64 : 128);
  p->nslot = p->N > 1 ? bit_length(p->N - 1) : 0;
  p->seg_log2 = seg_log2 >= 0 ? seg_log2 : auto_seg_log2(p->BH, dk, dv, C, p->N, p->L);
  p->nseg = p->N > 0 ? (p->N + (1 << p->seg_log2) - 1) >> p->seg_log2 : 0;
  p->blk_log2 = p->nseg > 1 ? auto_blk_log2(p->BH, dv, p->seg_log2, p->nseg) : p->seg_log2;
  p->nblk1 = ((p->nseg - 1) << (p->seg_log2 - p->blk_log2)) + 1;
  if (p->nseg > 1) {
    const size_t elems = (size_t)p->BH * dv * p->DKP;
    p->ws_state = align256(elems * p->nblk1 * sizeof(float));
    // fp32 node states, or (full-width sweep) the packed fp16 fragments and
    // exponents, which take less room
    p->ws_nodes = align256(std::max(elems * p->nseg * sizeof(float),
                                    ll::sweep_wide_ok(C, dk, dv, p->L, p->nslot, p->seg_log2)
                                        ? ll::node_pack_bytes(p->BH, p->nseg) : 0));
    p->ws_decay = align256((size_t)p->BH * p->nseg * sizeof(float));
    p->ws_bdecay = align256((size_t)p->BH * p->nblk1 * sizeof(float));
  } else {
    p->ws_state = p->ws_nodes = p->ws_decay = p->ws_bdecay = 0;
  }
  p->ws_total = p->ws_state + p->ws_nodes + p->ws_decay + p->ws_bdecay;
  return LL_OK;
}

int run_fwd(int dtype, const void* q, const void* k, const void* v, const float* log_a,
            const float* lambda, float* out, int B, int H, int T, int dk, int dv, int C,
            int seg_log2, int kernel, void* workspace, size_t workspace_bytes,
            void* const* events, const loglinear_states* fin, int qk_heads, hipStream_t stream,
            const ll::ScratchProvider* provider = nullptr) {
  FwdPlan p;
  int st = plan_fwd(B, H, T, dk, dv, C, seg_log2, &p);
  if (st != LL_OK) return st;
  const int G = heads_per_qk(H, qk_heads);
  if (G < 1) return LL_ERR_SHAPE;
  if (dtype != LL_BF16 && dtype != LL_F32) return LL_ERR_SHAPE;
  if (fin && (fin->N != B || fin->H != H || fin->dk != dk || fin->dv != dv || fin->L > 31 ||
              fin->L < (T > 0 ? p.L : 1)))
    return LL_ERR_SHAPE;
  if (B == 0 || H == 0 || T == 0) return LL_OK;
  if (!q || !k || !v || !log_a || !lambda || !out) return LL_ERR_NULL;
  if (fin && !fin->data) return LL_ERR_NULL;
  // Sweep kernel: the register-state kernel covers bf16, C = 64, 64 < dk <= 128,
  // dv a multiple of 64 and at most rs_max_slots() chunk-level Fenwick bits;
  // the LDS-state kernel covers everything else.
  const bool rs_ok = dtype == LL_BF16 && C == 64 && dk > 64 && dv % 64 == 0 &&
                     p.nslot <= ll::rs_max_slots() && p.L <= 17 &&
                     ll::rs_lds_bytes(p.L, p.nslot) <= ll::kMaxLds;
  const bool wide_ok = dtype == LL_BF16 && ll::sweep_wide_ok(C, dk, dv, p.L, p.nslot, p.seg_log2);
  if (kernel < LL_KERNEL_AUTO || kernel > LL_KERNEL_WIDE) return LL_ERR_SHAPE;
  if (kernel == LL_KERNEL_REGISTER_STATE && !rs_ok) return LL_ERR_UNSUPPORTED;
  if (kernel == LL_KERNEL_WIDE && !wide_ok) return LL_ERR_UNSUPPORTED;
  const bool use_wide = kernel == LL_KERNEL_WIDE || (kernel == LL_KERNEL_AUTO && kWideAuto && wide_ok);
  const bool use_rs = !use_wide && (kernel == LL_KERNEL_REGISTER_STATE || (kernel == LL_KERNEL_AUTO && rs_ok));
  if (!use_rs && !use_wide) {
    const int lds = ll::sweep_lds_bytes(dtype, C, p.DKP, p.L, p.nslot);
    if (lds < 0 || lds > ll::kMaxLds) return LL_ERR_UNSUPPORTED;
  }
  // a fixed-size scratch (allocation-free entry point): reject sizes beyond it
  // before any HIP call
  if (provider && p.ws_total > provider->max_bytes) return LL_ERR_WORKSPACE;
  if (workspace && workspace_bytes < p.ws_total) return LL_ERR_WORKSPACE;
  // the node states are read from the workspace as 16-byte vectors; the
  // header promises 256-byte alignment, which is what is checked
  if (workspace && (reinterpret_cast<uintptr_t>(workspace) & 255)) return LL_ERR_WORKSPACE;
  if (!aligned16({q, k, v, lambda, out, fin ? fin->data : nullptr})) return LL_ERR_SHAPE;

  void* ws = workspace;
  bool owned = false;
  if (p.ws_total > 0 && provider) {
    // every argument is checked: now the scratch's device address
    ws = provider->get();
    if (!ws) return LL_ERR_HIP;
  }
  if (p.ws_total > 0 && !ws) {
    if (hipMallocAsync(&ws, p.ws_total, stream) != hipSuccess) return LL_ERR_HIP;
    owned = true;
  }
  char* wsb = static_cast<char*>(ws);
  float* blk_state = reinterpret_cast<float*>(wsb);
  float* nodes = p.ws_total ? reinterpret_cast<float*>(wsb + p.ws_state) : nullptr;
  float* seg_decay = p.ws_total ? reinterpret_cast<float*>(wsb + p.ws_state + p.ws_nodes) : nullptr;
  float* blk_decay =
      p.ws_total ? reinterpret_cast<float*>(wsb + p.ws_state + p.ws_nodes + p.ws_decay) : nullptr;
  // the full-width sweep's packed nodes share the node region
  void* node16 = nodes;
  int* node_exp = p.ws_total ? reinterpret_cast<int*>(wsb + p.ws_state + (size_t)p.BH * p.nseg * 8 * 4 * 64 * 16)
                             : nullptr;

  auto mark = [&](int i) {
    if (events && st == LL_OK && hipEventRecord(static_cast<hipEvent_t>(events[i]), stream) != hipSuccess)
      st = LL_ERR_HIP;
  };
  mark(0);
  if (p.nseg > 1) {
    // block states: the state kernels see the blocks as segments, with one
    // unused slot at the end
    ll::SegArgs sa{k, v, log_a, blk_state, blk_decay, p.BH, T, dk, dv, C, p.blk_log2, p.nblk1, G};
    const int ndvg = (dv + 127) / 128;
    if (dtype == LL_BF16 && p.DKP == 128 && dv % 64 == 0)
      st = ll::launch_seg_state_rs(sa, p.BH, stream);
    else
      st = ll::launch_seg_state(dtype, p.DKP, sa, p.BH * (p.nblk1 - 1) * ndvg, stream);
    mark(1);
    if (st == LL_OK) {
      ll::NodeArgs na{blk_state, blk_decay, nodes, seg_decay, p.nseg, p.nblk1,
                      p.seg_log2 - p.blk_log2, dv * p.DKP};
      if (use_wide)
        st = ll::launch_node_pack(na, node16, node_exp, p.BH, stream);
      else
        st = ll::launch_seg_nodes(na, p.BH, stream);
    }
  } else {
    mark(1);
  }
  mark(2);
  if (st == LL_OK) {
    ll::FwdArgs fa{q, k, v, log_a, lambda, out, nodes, seg_decay, p.BH, T, dk, dv, p.L,
                   p.seg_log2, p.nseg, p.nslot, fin ? fin->data : nullptr, fin ? fin->L : 0, G,
                   node16, node_exp};
    const long long pairs = (long long)p.BH * p.nseg;
    const long long nblocks = ((pairs + 7) / 8) * 8 * (use_rs ? dv / 64 : dv / 16);
    if (use_wide) st = ll::launch_sweep_wide(fa, stream);
    else if (nblocks > 0x7fffffffLL) st = LL_ERR_UNSUPPORTED;
    else if (use_rs) st = ll::launch_sweep_rs(fa, static_cast<int>(nblocks), stream);
    else st = ll::launch_sweep(dtype, C, p.DKP, fa, static_cast<int>(nblocks), stream);
  }
  if (st == LL_OK && fin) {
    // levels 0..log2(C) of the prefill states; the sweep wrote the others
    ll::HandoffArgs ha{k, v, log_a, fin->data, p.BH, T, dk, dv, C, fin->L, G};
    st = ll::launch_handoff_intra(dtype, ha, stream);
  }
  mark(3);
  if (owned) {
    if (hipFreeAsync(ws, stream) != hipSuccess && st == LL_OK) st = LL_ERR_HIP;
  }
  return st;
}

int run_decode(int dtype, const loglinear_states* s, const void* q, const void* k, const void* v,
               const float* log_a, const float* lambda, const int* t, float* out, int qk_heads,
               hipStream_t stream) {
  if (!s) return LL_ERR_NULL;
  if (s->N < 0 || s->H < 0) return LL_ERR_SHAPE;
  if (dtype != LL_BF16 && dtype != LL_F32) return LL_ERR_SHAPE;
  const int G = s->H > 0 ? heads_per_qk(s->H, qk_heads) : 1;
  if (G < 1) return LL_ERR_SHAPE;
  if (s->L < 1 || s->L > 31) return LL_ERR_SHAPE;
  if (s->dk < 4 || s->dk % 4 != 0 || s->dv < 4 || s->dv % 4 != 0) return LL_ERR_SHAPE;
  if (s->dk > 1024 || s->dv > 1024) return LL_ERR_UNSUPPORTED;
  if ((long long)s->N * s->H > 0x7fffffffLL) return LL_ERR_UNSUPPORTED;
  if (s->N == 0 || s->H == 0) return LL_OK;
  if (!s->data || !q || !k || !v || !log_a || !lambda || !t || !out) return LL_ERR_NULL;
  // states and out move as 16-byte vectors; q, k, v are read one element at a time
  if (!aligned16({s->data, out})) return LL_ERR_SHAPE;
  ll::DecArgs a{s->data, q, k, v, log_a, lambda, t, out, s->N, s->H, s->L, s->dk, s->dv, G};
  return ll::launch_decode(dtype, a, stream);
}

int run_gdn_decode(int dtype, const loglinear_states* s, const void* q, const void* k, const void* v,
                   const float* log_alpha, const float* beta, const float* lambda, const int* t,
                   float* out, hipStream_t stream) {
  if (!s) return LL_ERR_NULL;
  if (s->N < 0 || s->H < 0) return LL_ERR_SHAPE;
  if (dtype != LL_BF16 && dtype != LL_F32) return LL_ERR_SHAPE;
  if (s->L < 1 || s->L > 31) return LL_ERR_SHAPE;
  if (s->dk < 4 || s->dk % 4 != 0 || s->dv < 4 || s->dv % 4 != 0) return LL_ERR_SHAPE;
  if ((s->dk != 64 && s->dk != 128) || s->dv > 1024) return LL_ERR_UNSUPPORTED;
  if ((long long)s->N * s->H > 0x7fffffffLL) return LL_ERR_UNSUPPORTED;
  if (s->N == 0 || s->H == 0) return LL_OK;
  if (!s->data || !q || !k || !v || !log_alpha || !beta || !lambda || !t || !out) return LL_ERR_NULL;
  // states and out move as 16-byte vectors; q, k, v are read one element at a time
  if (!aligned16({s->data, out})) return LL_ERR_SHAPE;
  ll::GdnDecArgs a{s->data, q, k, v, log_alpha, beta, lambda, t, out, s->N, s->H, s->L, s->dk, s->dv};
  return ll::launch_gdn_decode(dtype, a, stream);
}

int run_lambda_proj(int dtype, const void* x, const void* W, const float* bias, float* lam, int B, int T,
                    int D, int H, int L, hipStream_t stream) {
  if (dtype != LL_BF16 && dtype != LL_F32) return LL_ERR_SHAPE;
  if (B < 0 || T < 0 || D < 1 || H < 1 || L < 1 || L > 31) return LL_ERR_SHAPE;
  if (D % (dtype == LL_BF16 ? 8 : 4) != 0) return LL_ERR_SHAPE;  // 16-byte rows
  if (D > (1 << 20) || (long long)H * L > (1 << 20)) return LL_ERR_UNSUPPORTED;
  if ((long long)B * T > (1LL << 40)) return LL_ERR_UNSUPPORTED;
  if (B == 0 || T == 0) return LL_OK;
  if (!x || !W || !lam) return LL_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(W)) & 15) return LL_ERR_SHAPE;
  const int ncb = (H * L + 255) / 256;
  ll::LamProjArgs a{x, W, bias, lam, B, T, D, H, L, ncb};
  return ll::launch_lambda_proj(dtype, a, stream);
}

int run_lambda_proj_bwd(int dtype, const void* x, const void* W, const float* lam, const float* dlam,
                        float* dx, float* dW, float* dbias, int B, int T, int D, int H, int L,
                        hipStream_t stream) {
  if (dtype != LL_BF16 && dtype != LL_F32) return LL_ERR_SHAPE;
  if (B < 0 || T < 0 || D < 1 || H < 1 || L < 1 || L > 31) return LL_ERR_SHAPE;
  if (D > (1 << 20) || (long long)H * L > (1 << 16)) return LL_ERR_UNSUPPORTED;
  const long long M = (long long)B * T;
  if (M > 0x7fffffffLL) return LL_ERR_UNSUPPORTED;
  if (!W || !dW) return LL_ERR_NULL;
  if (M > 0 && (!x || !lam || !dlam || !dx)) return LL_ERR_NULL;
  const int HL = H * L;
  if (dtype == LL_BF16) {
    ll::LamBwdArgs a{x, W, lam, dlam, nullptr, dx, dW, dbias, B, T, D, H, L};
    ll::Lam16Plan p;
    if (ll::lambda_bwd16_plan(a, &p)) {
      void* ws = nullptr;
      if (hipMallocAsync(&ws, ll::lambda_bwd16_workspace(p), stream) != hipSuccess) return LL_ERR_HIP;
      int st = ll::launch_lambda_bwd16(a, p, ws, stream);
      if (hipFreeAsync(ws, stream) != hipSuccess && st == LL_OK) st = LL_ERR_HIP;
      return st;
    }
  }
  const int nsplit = M > 0 ? ll::lambda_bwd_nsplit(M, HL, D) : 0;
  const size_t dz_bytes = align256((size_t)M * HL * sizeof(float));
  const size_t part_bytes = align256((size_t)nsplit * HL * (D + 1) * sizeof(float));
  void* ws = nullptr;
  if (dz_bytes + part_bytes > 0 && hipMallocAsync(&ws, dz_bytes + part_bytes, stream) != hipSuccess)
    return LL_ERR_HIP;
  char* wsb = static_cast<char*>(ws);
  float* dz = reinterpret_cast<float*>(wsb);
  float* part = reinterpret_cast<float*>(wsb + dz_bytes);
  ll::LamBwdArgs a{x, W, lam, dlam, dz, dx, dW, dbias, B, T, D, H, L};
  int st = ll::launch_lambda_bwd(dtype, a, part, nsplit, stream);
  if (ws && hipFreeAsync(ws, stream) != hipSuccess && st == LL_OK) st = LL_ERR_HIP;
  return st;
}

// A second stream per device for the part of the backward that does not
// depend on the rest (the dQ chain runs beside the dK / dV chain, joined by an
// event before the kernels that need both).  Default priority; created on
// first use and kept until the process ends.  `mu` makes one call's
// fork/join sequence atomic with respect to other host threads, since the two
// events are shared.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  std::mutex mu;
};

SideStream* side_stream() {
  static SideStream ss[64];
  static std::mutex init_mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> g(init_mu);
  SideStream& x = ss[dev];
  if (!x.s) {
    hipStream_t s = nullptr;
    hipEvent_t f = nullptr, j = nullptr;
    if (hipStreamCreateWithFlags(&s, hipStreamNonBlocking) != hipSuccess) return nullptr;
    if (hipEventCreateWithFlags(&f, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&j, hipEventDisableTiming) != hipSuccess) {
      if (f) hipEventDestroy(f);
      hipStreamDestroy(s);
      return nullptr;
    }
    x.fork = f;
    x.join = j;
    x.s = s;
  }
  return &x;
}

int run_bwd(int dtype, const void* q, const void* k, const void* v, const float* log_a,
            const float* lambda, const float* out, const float* dout, float* dq, float* dk_out,
            float* dv_out, float* dlog_a, float* dlambda, int B, int H, int T, int dk, int dv, int C,
            int qk_heads, hipStream_t stream) {
  FwdPlan p;
  int st = plan_fwd(B, H, T, dk, dv, C, 0, &p);
  if (st != LL_OK) return st;
  if (dtype != LL_BF16 && dtype != LL_F32) return LL_ERR_SHAPE;
  const int G = heads_per_qk(H, qk_heads);
  if (G < 1) return LL_ERR_SHAPE;
  if (B == 0 || H == 0 || T == 0) return LL_OK;
  // `out` is not read (d log_a takes dO_t . O_t as sum_l lambda dlambda), so it may be NULL
  (void)out;
  if (!q || !k || !v || !log_a || !lambda || !dout || !dq || !dk_out || !dv_out || !dlog_a || !dlambda)
    return LL_ERR_NULL;
  if (p.nslot > 16 || p.N > 4096) return LL_ERR_UNSUPPORTED;
  const int lds = ll::bwd_lds_bytes(dtype, C, dk, dv, p.L, p.N, p.nslot);
  if (lds > ll::kMaxLds) return LL_ERR_UNSUPPORTED;
  if (!aligned16({q, k, v, lambda, dout, dq, dk_out, dv_out, dlambda})) return LL_ERR_SHAPE;
  const size_t part = align256((size_t)(dk / 16) * p.BH * T * (p.nslot > 0 ? p.nslot : 1) * sizeof(float));
  const size_t dcb = align256((size_t)p.BH * T * sizeof(double));
  // shared q / k: per-head gradients first, then summed over each group
  const size_t per_head = G > 1 ? align256((size_t)p.BH * T * dk * sizeof(float)) : 0;
  // dQ through the register-state forward sweep run on (dO, v, k): dQ_t =
  // sum_s M[t,s] (dO_t . v_s) k_s is the forward with q, k, v taken as dO, v,
  // k, and the same sweep forms the chunk-level dlambda (the dot of each
  // level's read with q).  Its variant reads dO in fp32 and runs the score
  // tiles and the level reads on fp16 with a per-row power-of-two scale (one
  // bf16 rounding of dO measured up to 3e-2 of the RMS).  Shapes: bf16,
  // C = 64, q / k per head, the register-state sweep's (contraction dv in
  // (64, 128], dk a multiple of 64, at most 256 chunks).
  FwdPlan pd{};
  bool dq_rs = dtype == LL_BF16 && C == 64 && G == 1 && dv > 64 && dv <= 128 && dk % 64 == 0 &&
               p.nslot <= 8;
  if (dq_rs) dq_rs = plan_fwd(B, H, T, dv, dk, C, -1, &pd) == LL_OK &&
                     ll::rs_dlam_lds_bytes(pd.L, pd.nslot) <= ll::kMaxLds;
  const size_t fws = dq_rs ? pd.ws_total : 0;
  // dV and dK through the reverse register-state sweep (bf16, C = 64,
  // dk = dv = 128, q / k per head); its pre-pass states follow the rest of
  // the workspace
  const bool kv_rev = dtype == LL_BF16 && ll::bwd_rev_ok(C, dk, dv, G, T, p.L);
  const size_t rws = kv_rev ? align256(ll::bwd_rev_workspace(p.BH, T)) : 0;
  // the dV sweep's row records (in-chunk dlambda and v . dV), one per
  // 64-column group of dv, and the 64-row block totals of dc
  const size_t iws = kv_rev ? align256((size_t)(dv / 64) * p.BH * T * 8 * sizeof(float)) : 0;
  const size_t bws = kv_rev ? align256((size_t)p.BH * ((T + 63) / 64) * sizeof(double)) : 0;
  void* ws = nullptr;
  if (hipMallocAsync(&ws, part + dcb + 2 * per_head + fws + rws + iws + bws, stream) != hipSuccess)
    return LL_ERR_HIP;
  char* wsb = static_cast<char*>(ws);
  float* dq_h = G > 1 ? reinterpret_cast<float*>(wsb + part + dcb) : dq;
  float* dk_h = G > 1 ? reinterpret_cast<float*>(wsb + part + dcb + per_head) : dk_out;
  ll::BwdArgs a{q, k, v, log_a, lambda, out, dout, dq_h, dk_h, dv_out, dlog_a, dlambda,
                reinterpret_cast<float*>(wsb), reinterpret_cast<double*>(wsb + part),
                p.BH, T, dk, dv, p.L, p.nslot, G};
  // the dQ chain on the side stream when the dK / dV chain runs too
  SideStream* side = dq_rs && kv_rev ? side_stream() : nullptr;
  std::unique_lock<std::mutex> side_lock;
  hipStream_t qs = stream;
  if (side) {
    side_lock = std::unique_lock<std::mutex>(side->mu);
    if (hipEventRecord(side->fork, stream) == hipSuccess && hipStreamWaitEvent(side->s, side->fork, 0) == hipSuccess)
      qs = side->s;
  }
  if (dq_rs) {
    char* fw = wsb + part + dcb + 2 * per_head;
    float* blk_state = reinterpret_cast<float*>(fw);
    float* nodes = pd.ws_total ? reinterpret_cast<float*>(fw + pd.ws_state) : nullptr;
    float* seg_decay = pd.ws_total ? reinterpret_cast<float*>(fw + pd.ws_state + pd.ws_nodes) : nullptr;
    float* blk_decay = pd.ws_total ? reinterpret_cast<float*>(fw + pd.ws_state + pd.ws_nodes + pd.ws_decay) : nullptr;
    if (pd.nseg > 1) {
      // segment states of the swapped problem: keys v, values k
      ll::SegArgs sa{v, k, log_a, blk_state, blk_decay, pd.BH, T, dv, dk, C, pd.blk_log2, pd.nblk1, 1};
      st = ll::launch_seg_state_rs(sa, pd.BH, qs);
      if (st == LL_OK) {
        ll::NodeArgs na{blk_state, blk_decay, nodes, seg_decay, pd.nseg, pd.nblk1, pd.seg_log2 - pd.blk_log2,
                        dk * pd.DKP};
        st = ll::launch_seg_nodes(na, pd.BH, qs);
      }
    }
    const long long pairs = (long long)pd.BH * pd.nseg;
    const long long nblocks = ((pairs + 7) / 8) * 8 * (dk / 64);
    if (nblocks > 0x7fffffffLL) st = LL_ERR_UNSUPPORTED;
    if (st == LL_OK) {
      ll::FwdArgs fa{dout, v, k, log_a, lambda, dq_h, nodes, seg_decay, pd.BH, T, dv, dk, pd.L,
                     pd.seg_log2, pd.nseg, pd.nslot, nullptr, 0, 1};
      fa.qo = q;
      fa.dlam_part = a.dlam_part;
      st = ll::launch_sweep_rs_dlam(fa, static_cast<int>(nblocks), qs);
    }
    a.dq_done = 1;
    a.dlam_parts = dk / 64;
  }
  if (st == LL_OK && kv_rev) {
    ll::BwdRevPlan rp;
    ll::bwd_rev_plan(T, &rp);
    char* rw = wsb + part + dcb + 2 * per_head + fws;
    float* seg_part = rws ? reinterpret_cast<float*>(rw) : nullptr;
    float* seg_tot2 =
        rws ? reinterpret_cast<float*>(rw + (size_t)p.BH * rp.nseg * rp.nj * dk * dv * sizeof(float)) : nullptr;
    ll::BwdRevArgs ra{q, k, v, dout, log_a, lambda, dk_h, dv_out, seg_part, seg_tot2,
                      p.BH, T, p.L, rp.seg_log2, rp.nseg, rp.nj};
    ra.intra_part = reinterpret_cast<float*>(wsb + part + dcb + 2 * per_head + fws + rws);
    st = ll::launch_bwd_rev(ra, stream);
    a.kv_done = 1;
    a.dlam_intra_part = ra.intra_part;
    a.intra_parts = dv / 64;
    a.dc_blk = reinterpret_cast<double*>(wsb + part + dcb + 2 * per_head + fws + rws + iws);
  }
  // join: whatever was enqueued on the side stream finishes before the main
  // stream goes on (also after an error, before the workspace is freed)
  if (qs != stream && (hipEventRecord(side->join, qs) != hipSuccess ||
                       hipStreamWaitEvent(stream, side->join, 0) != hipSuccess)) {
    if (st == LL_OK) st = LL_ERR_HIP;
    hipStreamSynchronize(qs);
  }
  if (st == LL_OK) st = ll::launch_bwd(dtype, C, a, stream);
  if (st == LL_OK && G > 1) {
    const long long rows = (long long)p.BH / G, elems = (long long)T * dk;
    st = ll::launch_group_sum(dq_h, dq, rows, G, elems, stream);
    if (st == LL_OK) st = ll::launch_group_sum(dk_h, dk_out, rows, G, elems, stream);
  }
  if (hipFreeAsync(ws, stream) != hipSuccess && st == LL_OK) st = LL_ERR_HIP;
  return st;
}

int gdn_plan(int B, int H, int T, int dk, int dv, int* N, int* nslot, size_t* ws) {
  if (B < 0 || H < 0 || T < 0 || dk <= 0 || dv <= 0) return LL_ERR_SHAPE;
  if (dk != 64 && dk != 128) return LL_ERR_UNSUPPORTED;
  if (dv % 16 != 0) return LL_ERR_UNSUPPORTED;
  *N = (T + 63) / 64;
  *nslot = *N > 1 ? bit_length(*N - 1) : 0;
  if (ll::gdn_sweep_lds_bytes(*nslot, dk) > ll::kMaxLds) return LL_ERR_UNSUPPORTED;
  *ws = ll::gdn_workspace_bytes((long long)B * H, *N, dk);
  return LL_OK;
}

int run_gdn(int dtype, const void* q, const void* k, const void* v, const float* log_alpha,
            const float* beta, const float* lambda, float* out, int B, int H, int T, int dk, int dv,
            void* workspace, size_t workspace_bytes, hipStream_t stream, float* st_out = nullptr,
            int st_L = 0) {
  int N = 0, nslot = 0;
  size_t need = 0;
  if (dtype != LL_BF16 && dtype != LL_F32) return LL_ERR_SHAPE;
  int st = gdn_plan(B, H, T, dk, dv, &N, &nslot, &need);
  if (st != LL_OK) return st;
  const int L = T > 0 ? bit_length(T - 1) + 1 : 0;
  if (st_out && (st_L < std::max(L, 1) || st_L > 31)) return LL_ERR_SHAPE;
  if (B == 0 || H == 0 || T == 0) return LL_OK;
  if (!q || !k || !v || !log_alpha || !beta || !lambda || !out) return LL_ERR_NULL;
  if (!aligned16({q, k, v, lambda, out, st_out})) return LL_ERR_SHAPE;
  if (workspace && workspace_bytes < need) return LL_ERR_WORKSPACE;
  if (workspace && (reinterpret_cast<uintptr_t>(workspace) & 255)) return LL_ERR_WORKSPACE;
  void* ws = workspace;
  bool owned = false;
  if (!ws) {
    if (hipMallocAsync(&ws, need, stream) != hipSuccess) return LL_ERR_HIP;
    owned = true;
  }
  const long long BH = (long long)B * H;
  const size_t rec_bytes = need - align256(size_t(BH) * N * 4);
  ll::GdnArgs a{q, k, v, log_alpha, beta, lambda, out, static_cast<float*>(ws),
                reinterpret_cast<float*>(static_cast<char*>(ws) + rec_bytes),
                static_cast<int>(BH), T, dk, dv, L, N, nslot};
  a.st_out = st_out;
  a.st_L = st_L;
  st = ll::launch_gdn(dtype, a, stream);
  if (owned && hipFreeAsync(ws, stream) != hipSuccess && st == LL_OK) st = LL_ERR_HIP;
  return st;
}

}  // namespace

namespace ll {
int fwd_bf16_with_scratch(const void* q, const void* k, const void* v, const float* log_a,
                          const float* lambda, float* out, int B, int H, int T, int dk, int dv, int C,
                          const ScratchProvider& provider, hipStream_t stream) {
  return run_fwd(LL_BF16, q, k, v, log_a, lambda, out, B, H, T, dk, dv, C, -1, LL_KERNEL_AUTO, nullptr, 0,
                 nullptr, nullptr, 0, stream, &provider);
}
}  // namespace ll

extern "C" {

int loglinear_num_levels(int T) { return T >= 1 ? bit_length(T - 1) + 1 : 0; }

int loglinear_fwd(const void* q, const void* k, const void* v, const float* log_a,
                  const float* lambda, float* out, int B, int H, int T, int dk, int dv, int C,
                  void* stream) {
  return run_fwd(LL_BF16, q, k, v, log_a, lambda, out, B, H, T, dk, dv, C, -1, LL_KERNEL_AUTO, nullptr, 0, nullptr,
                 nullptr, 0, static_cast<hipStream_t>(stream));
}

int loglinear_fwd_f32(const float* q, const float* k, const float* v, const float* log_a,
                      const float* lambda, float* out, int B, int H, int T, int dk, int dv, int C,
                      void* stream) {
  return run_fwd(LL_F32, q, k, v, log_a, lambda, out, B, H, T, dk, dv, C, -1, LL_KERNEL_AUTO, nullptr, 0, nullptr,
                 nullptr, 0, static_cast<hipStream_t>(stream));
}

int loglinear_prefill(const void* q, const void* k, const void* v, const float* log_a,
                      const float* lambda, float* out, const loglinear_states* states, int B,
                      int H, int T, int dk, int dv, int C, void* stream) {
  if (!states) return LL_ERR_NULL;
  return run_fwd(LL_BF16, q, k, v, log_a, lambda, out, B, H, T, dk, dv, C, -1, LL_KERNEL_AUTO, nullptr, 0, nullptr,
                 states, 0, static_cast<hipStream_t>(stream));
}

int loglinear_prefill_f32(const float* q, const float* k, const float* v, const float* log_a,
                          const float* lambda, float* out, const loglinear_states* states,
                          int B, int H, int T, int dk, int dv, int C, void* stream) {
  if (!states) return LL_ERR_NULL;
  return run_fwd(LL_F32, q, k, v, log_a, lambda, out, B, H, T, dk, dv, C, -1, LL_KERNEL_AUTO, nullptr, 0, nullptr,
                 states, 0, static_cast<hipStream_t>(stream));
}

int loglinear_fwd_ex(const void* q, const void* k, const void* v, const float* log_a,
                     const float* lambda, float* out, int B, int H, int T, int dk, int dv, int C,
                     const loglinear_fwd_opts* opts, void* stream) {
  if (!opts) return LL_ERR_NULL;
  return run_fwd(opts->dtype, q, k, v, log_a, lambda, out, B, H, T, dk, dv, C, opts->seg_log2,
                 opts->kernel, opts->workspace, opts->workspace_bytes, opts->phase_events,
                 opts->final_states, opts->qk_heads, static_cast<hipStream_t>(stream));
}

int loglinear_bwd(const void* q, const void* k, const void* v, const float* log_a,
                  const float* lambda, const float* out, const float* dout, float* dq, float* dk_out,
                  float* dv_out, float* dlog_a, float* dlambda, int B, int H, int T, int dk, int dv,
                  int C, void* stream) {
  return run_bwd(LL_BF16, q, k, v, log_a, lambda, out, dout, dq, dk_out, dv_out, dlog_a, dlambda, B, H, T,
                 dk, dv, C, 0, static_cast<hipStream_t>(stream));
}

int loglinear_bwd_f32(const float* q, const float* k, const float* v, const float* log_a,
                      const float* lambda, const float* out, const float* dout, float* dq,
                      float* dk_out, float* dv_out, float* dlog_a, float* dlambda, int B, int H, int T,
                      int dk, int dv, int C, void* stream) {
  return run_bwd(LL_F32, q, k, v, log_a, lambda, out, dout, dq, dk_out, dv_out, dlog_a, dlambda, B, H, T,
                 dk, dv, C, 0, static_cast<hipStream_t>(stream));
}

int loglinear_bwd_ex(const void* q, const void* k, const void* v, const float* log_a,
                     const float* lambda, const float* out, const float* dout, float* dq,
                     float* dk_out, float* dv_out, float* dlog_a, float* dlambda, int B, int H, int T,
                     int dk, int dv, int C, int dtype, int qk_heads, void* stream) {
  return run_bwd(dtype, q, k, v, log_a, lambda, out, dout, dq, dk_out, dv_out, dlog_a, dlambda, B, H, T,
                 dk, dv, C, qk_heads, static_cast<hipStream_t>(stream));
}

int loglinear_lambda_proj(const void* x, const void* W, const float* bias, float* lambda, int B, int T,
                          int D, int H, int L, int dtype, void* stream) {
  return run_lambda_proj(dtype, x, W, bias, lambda, B, T, D, H, L, static_cast<hipStream_t>(stream));
}

int loglinear_lambda_proj_bwd(const void* x, const void* W, const float* lambda,
                              const float* grad_lambda, float* grad_x, float* grad_W,
                              float* grad_bias, int B, int T, int D, int H, int L, int dtype,
                              void* stream) {
  return run_lambda_proj_bwd(dtype, x, W, lambda, grad_lambda, grad_x, grad_W, grad_bias, B, T, D, H, L,
                             static_cast<hipStream_t>(stream));
}

size_t loglinear_fwd_workspace_size(int B, int H, int T, int dk, int dv, int C, int seg_log2) {
  FwdPlan p;
  if (plan_fwd(B, H, T, dk, dv, C, seg_log2, &p) != LL_OK) return static_cast<size_t>(-1);
  return p.ws_total;
}

int loglinear_decode_step(const loglinear_states* states, const void* q, const void* k,
                          const void* v, const float* log_a, const float* lambda, const int* t,
                          float* out, void* stream) {
  return run_decode(LL_BF16, states, q, k, v, log_a, lambda, t, out, 0,
                    static_cast<hipStream_t>(stream));
}

int loglinear_decode_step_f32(const loglinear_states* states, const float* q, const float* k,
                              const float* v, const float* log_a, const float* lambda,
                              const int* t, float* out, void* stream) {
  return run_decode(LL_F32, states, q, k, v, log_a, lambda, t, out, 0,
                    static_cast<hipStream_t>(stream));
}

int loglinear_decode_step_ex(const loglinear_states* states, const void* q, const void* k,
                             const void* v, const float* log_a, const float* lambda, const int* t,
                             float* out, int dtype, int qk_heads, void* stream) {
  return run_decode(dtype, states, q, k, v, log_a, lambda, t, out, qk_heads,
                    static_cast<hipStream_t>(stream));
}

int loglinear_gdn_fwd(const void* q, const void* k, const void* v, const float* log_alpha,
                      const float* beta, const float* lambda, float* out, int B, int H, int T, int dk,
                      int dv, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return run_gdn(dtype, q, k, v, log_alpha, beta, lambda, out, B, H, T, dk, dv, workspace,
                 workspace_bytes, static_cast<hipStream_t>(stream));
}

int loglinear_gdn_prefill(const void* q, const void* k, const void* v, const float* log_alpha,
                          const float* beta, const float* lambda, float* out, float* states,
                          int states_L, int B, int H, int T, int dk, int dv, int dtype, void* workspace,
                          size_t workspace_bytes, void* stream) {
  if (!states && B > 0 && H > 0 && T > 0) return LL_ERR_NULL;
  return run_gdn(dtype, q, k, v, log_alpha, beta, lambda, out, B, H, T, dk, dv, workspace,
                 workspace_bytes, static_cast<hipStream_t>(stream), states, states ? states_L : 0);
}

int loglinear_gdn_decode_step(const loglinear_states* states, const void* q, const void* k,
                              const void* v, const float* log_alpha, const float* beta,
                              const float* lambda, const int* t, float* out, int dtype, void* stream) {
  return run_gdn_decode(dtype, states, q, k, v, log_alpha, beta, lambda, t, out,
                        static_cast<hipStream_t>(stream));
}

size_t loglinear_gdn_workspace_size(int B, int H, int T, int dk, int dv) {
  int N = 0, nslot = 0;
  size_t ws = 0;
  if (gdn_plan(B, H, T, dk, dv, &N, &nslot, &ws) != LL_OK) return static_cast<size_t>(-1);
  return ws;
}

int loglinear_level_table(signed char* lev, int T, void* stream) {
  if (T < 1 || T > 8192) return LL_ERR_SHAPE;
  if (!lev) return LL_ERR_NULL;
  return ll::launch_level_table(lev, T, static_cast<hipStream_t>(stream));
}

const char* loglinear_strerror(int status) {
  switch (status) {
    case LL_OK: return "success";
    case LL_ERR_NULL: return "a required pointer is NULL";
    case LL_ERR_SHAPE: return "a size is negative, inconsistent or out of range";
    case LL_ERR_UNSUPPORTED: return "sizes are valid but no kernel of this build supports them";
    case LL_ERR_HIP: return "a HIP runtime call failed";
    case LL_ERR_WORKSPACE:
      return "workspace too small or misaligned (caller workspace, or the static scratch of "
             "loglinear_fwd_noalloc)";
    default: return "unknown status";
  }
}

}  // extern "C"
