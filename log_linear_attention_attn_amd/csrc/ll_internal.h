// Internal interfaces between the C ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

#include "loglinear.h"

namespace ll {

// Largest dynamic LDS allocation of one workgroup on gfx950 (160 KiB per CU).
constexpr int kMaxLds = 160 * 1024;

// Raises a kernel's dynamic LDS limit (default kMaxLds, less for kernels
// with static LDS) once per (kernel, device): `done` is the kernel's own bit
// set of devices already raised.
inline bool raise_lds_limit(const void* fn, std::atomic<uint64_t>& done, int bytes = kMaxLds) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  const uint64_t bit = dev >= 0 && dev < 64 ? uint64_t(1) << dev : 0;
  if (bit && (done.load(std::memory_order_relaxed) & bit)) return true;
  if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes) != hipSuccess) return false;
  done.fetch_or(bit, std::memory_order_relaxed);
  return true;
}

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* log_a;
  const float* lam;
  float* out;
  const float* nodes;      // [BH][nseg][dv][DKP] bucket states starting at each segment
  const float* seg_decay;  // [BH][nseg] total log decay of each segment
  int BH, T, dk, dv, L;
  int seg_log2;  // chunks per segment = 2^seg_log2
  int nseg;
  int nslot;  // chunk-level Fenwick bits = bit_length(N - 1)
  // Decode states at position T-1 (prefill), or null: [BH][st_L][dk][dv] fp32.
  // The sweep's last segment writes the inter-chunk levels log2(C)+1 .. st_L-1.
  float* st_out;
  int st_L;
  int G = 1;  // heads per q/k head: q and k of head bh are row bh / G
  // full-width sweep: the segment-spanning bucket states as fp16 MFMA
  // fragments [BH][nseg][8 waves][4][64 lanes] x 16 bytes, and their
  // power-of-two exponents [BH][nseg][8 waves] (node_pack_kernel)
  const void* node16 = nullptr;
  const int* node_exp = nullptr;
  // backward use (dQ as the forward of (dO, v, k)): the forward's own q
  // [BH][T][dv] bf16 and the chunk-level dlambda partials
  // [dv / 64][BH][T][nslot] this sweep writes (one part per 64-column group)
  const void* qo = nullptr;
  float* dlam_part = nullptr;
};

struct HandoffArgs {
  const void* k;
  const void* v;
  const float* log_a;
  float* st_out;  // [BH][st_L][dk][dv]
  int BH, T, dk, dv, C, st_L;
  int G = 1;  // heads per q/k head: q and k of head bh are row bh / G
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* log_a;
  const float* lam;
  const float* out;    // forward output (for the decay gradient)
  const float* dout;   // gradient of the loss with respect to out
  float* dq;           // [BH][T][dk]
  float* dk_out;       // [BH][T][dk]
  float* dvo;          // [BH][T][dv]
  float* dlog_a;       // [BH][T]
  float* dlam;         // [BH][T][L]
  float* dlam_part;    // [dk/16][BH][T][nslot] chunk-level dlam partial sums
  double* dc;          // [BH][T] dO.O - v.dV per token
  int BH, T, dk, dv, L;
  int nslot;           // chunk-level Fenwick bits = bit_length(N - 1)
  int G = 1;  // heads per q/k head: q and k of head bh are row bh / G
  // dQ and the chunk-level dlambda partials already formed by the
  // register-state sweep (launch_sweep_rs_dlam): the backward then skips its
  // own dQ sweep and sums dlam_parts partials per (t, level)
  int dq_done = 0;
  int dlam_parts = 0;
  // dK and dV already formed by the reverse register-state sweep
  // (launch_bwd_rev): the backward skips its own
  int kv_done = 0;
  // the reverse sweeps' per-row records ([intra_parts][BH][T][8]: the
  // in-chunk dlambda in words 0..6, v . dV in word 7): the backward forms
  // dlam and dc from them in one pass, and then needs dc_blk, the totals of
  // dc over each 64-row block of a (b,h) ([BH][ceil(T / 64)])
  const float* dlam_intra_part = nullptr;
  int intra_parts = 0;
  double* dc_blk = nullptr;
};

// Reverse register-state sweep for dV and dK (bf16, C = 64, dk = dv = 128,
// q / k per head): chunks of 2^seg_log2 per segment; the pre-pass writes the
// per-(segment, level) states seg_part [BH][nseg][nj][128][128] fp32 and the
// segments' log2 decay totals seg_tot2 [BH][nseg] (workspace, nseg > 1 only).
struct BwdRevArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* dout;
  const float* log_a;
  const float* lam;
  float* dk_out;  // [BH][T][128]
  float* dv_out;  // [BH][T][128]
  float* seg_part;
  float* seg_tot2;
  int BH, T, L, seg_log2, nseg, nj;
  // the dV sweep's in-chunk dlambda partials [2 column groups][BH][T][8]
  // (levels 0 .. log2C in the first seven words), or null
  float* intra_part = nullptr;
};
struct BwdRevPlan {
  int seg_log2, nseg, nj;
};
void bwd_rev_plan(int T, BwdRevPlan* p);
bool bwd_rev_ok(int C, int dk, int dv, int G, int T, int L);
size_t bwd_rev_workspace(int BH, int T);
int launch_bwd_rev(const BwdRevArgs& a, hipStream_t s);

struct SegArgs {
  const void* k;
  const void* v;
  const float* log_a;
  float* seg_state;  // [BH][nseg][dv][DKP]
  float* seg_decay;  // [BH][nseg]
  int BH, T, dk, dv, C, seg_log2, nseg;
  int G = 1;  // heads per q/k head: q and k of head bh are row bh / G
};

// Segment states are built from blocks of 2^blk_log2 chunks (a segment holds
// 2^rlog2 blocks), so that the state kernel has enough workgroups.
struct NodeArgs {
  const float* blk_state;  // [BH][nblk1][dv][DKP] decayed k v^T sum of each block
  const float* blk_decay;  // [BH][nblk1] total log decay of each block
  float* nodes;            // [BH][nseg][dv][DKP]
  float* seg_decay;        // [BH][nseg] total log decay of each segment (all but the last)
  int nseg;
  int nblk1;  // block slots per (b,h) = blocks of the first nseg - 1 segments + 1
  int rlog2;  // blocks per segment = 2^rlog2
  int E;      // elements per state = dv * DKP
};

struct DecArgs {
  float* S;
  const void* q;
  const void* k;
  const void* v;
  const float* log_a;
  const float* lam;
  const int* t;
  float* out;
  int N, H, L, dk, dv;
  int G = 1;  // heads per q/k head: q and k of head bh are row bh / G
};

struct LamProjArgs {
  const void* x;      // [B][T][D]
  const void* W;      // [H*L][D]
  const float* bias;  // [H*L] or null
  float* lam;         // [B][H][T][L]
  int B, T, D, H, L;
  int ncb;  // column blocks of 256 output columns
};

// Gradient of the level-weight projection.
struct LamBwdArgs {
  const void* x;      // [B][T][D]
  const void* W;      // [H*L][D]
  const float* lam;   // [B][H][T][L], the forward's output
  const float* dlam;  // [B][H][T][L]
  float* dz;          // scratch [B*T][H*L]
  float* dx;          // [B][T][D]
  float* dW;          // [H*L][D]
  float* dbias;       // [H*L] or null
  int B, T, D, H, L;
};

// C(m, n) = sum_{k in split} A(m, k) B(k, n) for the split given by the
// workgroup, written at C + split * split_stride + m * ldc + n; A(m, k) =
// A[m * sam + k * sak], B(k, n) = B[k * sbk + n * sbn] for n < nb_real, and
// for n >= nb_real 1 (n == nb_real with ones set) or 0.
struct GemmArgs {
  const void* A;
  const void* B;
  float* C;
  long long sam, sak, sbk, sbn, ldc, split_stride;
  int M, N, K, kper, nb_real, ones;
};

// A workspace of fixed size that is not allocated per call: max_bytes bounds
// it, get() returns its device address (null on a HIP error) and is called
// only after every argument has been checked.
struct ScratchProvider {
  size_t max_bytes;
  void* (*get)();
};
// loglinear_fwd with the workspace taken from `provider` (no allocation).
int fwd_bf16_with_scratch(const void* q, const void* k, const void* v, const float* log_a,
                          const float* lambda, float* out, int B, int H, int T, int dk, int dv, int C,
                          const ScratchProvider& provider, hipStream_t stream);

int sweep_lds_bytes(int dtype, int C, int DKP, int L, int nslot);
int launch_sweep(int dtype, int C, int DKP, const FwdArgs& a, int nblocks, hipStream_t s);
int launch_seg_state(int dtype, int DKP, const SegArgs& a, int nblocks, hipStream_t s);
int launch_seg_nodes(const NodeArgs& a, int BH, hipStream_t s);
// full-width register-state sweep (bf16, C = 64, 64 < dk <= 128, dv = 128,
// at most 8 chunk-level bits): one workgroup per (b,h, segment)
bool sweep_wide_ok(int C, int dk, int dv, int L, int nslot, int seg_log2);
// segment sizes the full-width sweep is built for (2^seg_log2 chunks)
bool sweep_wide_seg_ok(int seg_log2, int nslot);
int launch_sweep_wide(const FwdArgs& a, hipStream_t s);
// packed node states for the full-width sweep (node16 / node_exp of FwdArgs),
// plus the segments' total log decays; bytes of workspace they take
size_t node_pack_bytes(int BH, int nseg);
int launch_node_pack(const NodeArgs& a, void* node16, int* node_exp, int BH, hipStream_t s);
int rs_max_slots();
// dQ of the backward as the forward of (dO in fp32, v, k) plus the chunk-level
// dlambda partials (FwdArgs::qo, dlam_part); register-state shapes only
int launch_sweep_rs_dlam(const FwdArgs& a, int nblocks, hipStream_t stream);
int rs_dlam_lds_bytes(int L, int nslot);
int rs_lds_bytes(int L, int nslot);
int launch_sweep_rs(const FwdArgs& a, int nblocks, hipStream_t s);
int launch_seg_state_rs(const SegArgs& a, int BH, hipStream_t s);
int launch_level_table(signed char* lev, int T, hipStream_t s);
// Log-linear Gated DeltaNet forward: chunk records, then the level sweep.
struct GdnArgs {
  const void* q;          // [BH][T][dk]
  const void* k;          // [BH][T][dk]
  const void* v;          // [BH][T][dv]
  const float* log_alpha; // [BH][T]
  const float* beta;      // [BH][T]
  const float* lam;       // [BH][T][L]
  float* out;             // [BH][T][dv]
  float* ws;              // per-chunk records [BH][N] x gdn chunk record
  float* gchunk;          // [BH][N] decay of each whole chunk
  int BH, T, dk, dv, L, N;
  int nslot;              // chunk-level Fenwick bits = bit_length(N - 1)
  // decode states at position T-1 (prefill), or null: [BH][st_L][dk][dv] fp32
  float* st_out = nullptr;
  int st_L = 0;
};
size_t gdn_workspace_bytes(long long BH, int N, int dk);
int gdn_sweep_lds_bytes(int nslot, int dk);
int launch_gdn(int dtype, const GdnArgs& a, hipStream_t s);
// Log-linear Gated DeltaNet decode step (states updated in place).
struct GdnDecArgs {
  float* S;               // [N][H][L][dk][dv]
  const void* q;          // [N][H][dk]
  const void* k;          // [N][H][dk]
  const void* v;          // [N][H][dv]
  const float* log_alpha; // [N][H]
  const float* beta;      // [N][H]
  const float* lam;       // [N][H][L]
  const int* t;           // [N]
  float* out;             // [N][H][dv]
  int N, H, L, dk, dv;
};
int launch_gdn_decode(int dtype, const GdnDecArgs& a, hipStream_t s);
int launch_handoff_intra(int dtype, const HandoffArgs& a, hipStream_t s);
int launch_decode(int dtype, const DecArgs& a, hipStream_t s);
int bwd_lds_bytes(int dtype, int C, int dk, int dv, int L, int N, int nslot);
int launch_bwd(int dtype, int C, const BwdArgs& a, hipStream_t s);
// dV / dK reverse sweep on bf16 matrix cores (bf16 inputs, C = 64)
bool bwd_kv16_ok(const BwdArgs& a);
int launch_bwd_kv16(const BwdArgs& a, hipStream_t s);
// dQ / chunk-level dlambda forward sweep on bf16 matrix cores (bf16 inputs, C = 64)
bool bwd_dq16_ok(const BwdArgs& a);
int launch_bwd_dq16(const BwdArgs& a, hipStream_t s);
// in-chunk dlambda on bf16 matrix cores (bf16 inputs, C = 64)
bool bwd_dlam_intra16_ok(const BwdArgs& a);
int launch_bwd_dlam_intra16(const BwdArgs& a, hipStream_t s);
int lambda_proj_lds_bytes(int dtype);
int launch_lambda_proj(int dtype, const LamProjArgs& a, hipStream_t s);
// split count and rows per split of the dW product, and the launch
// (part: nsplit * H*L * (D + 1) floats of scratch)
int lambda_bwd_nsplit(long long rows, int HL, int D);
long long lambda_bwd_kper(long long rows, int nsplit);
int launch_lambda_bwd(int dtype, const LamBwdArgs& a, float* part, int nsplit, hipStream_t s);
// bf16 inputs with D % 8 == 0 and 16-byte aligned x, W: dz split once into bf16
// hi / lo, both products on bf16 matrix cores.  plan() returns false where the
// path does not apply (then launch_lambda_bwd serves the call).
struct Lam16Plan {
  int HLp, nsplit, ntb;
  long long kper;
  size_t dz_bytes, colsum_bytes, part_bytes;
};
bool lambda_bwd16_plan(const LamBwdArgs& a, Lam16Plan* p);
size_t lambda_bwd16_workspace(const Lam16Plan& p);
int launch_lambda_bwd16(const LamBwdArgs& a, const Lam16Plan& p, void* ws, hipStream_t s);
// out[i][e] = sum_{g < G} in[i * G + g][e] for i < rows, e < elems (elems % 4 == 0)
int launch_group_sum(const float* in, float* out, long long rows, int G, long long elems, hipStream_t s);

}  // namespace ll
