// Internal interface between the C-ABI host library (kvm_api.cpp) and the
// gfx950 kernels (kvm_kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kvm {

constexpr int kHeadDim = 64;   // head dimension
constexpr int kRopeDims = 32;  // rotary dims [0,32)
constexpr int kLive = 32;      // live state-key dims [32,64)

// Sizes fixed at state creation.
struct Dims {
  int BH;             // sequences (batch * heads)
  int C;              // chunk
  int W;              // window
  int R;              // ring slots = W + C
  int ns;             // sinks
  int S_cap;          // most rows a state can reach
  int J_cap;          // most chunks a state can absorb
  int64_t V_cap;      // row versions per sequence (<= J_cap * C)
  int64_t idx_total;  // index-list entries per sequence (sum over j of rows after chunk j)
  int64_t max_tokens;
  float scale;        // softmax scale
  float ln_eps;
  int bf16;           // 1: bf16 storage and MFMA; 0: fp32
  int trace;          // 1: record per-token assignment
  int no_vnorm;       // 1: read values as the mean V/n (ablation)
  int unprot;         // 1: sink rows are ordinary rows (ablation)
  int no_gate;        // 1: merge weight 1 (ablation)
  int P;              // scan workgroups per sequence (1, 2, 4 or 8); each owns every P-th 32-row tile
                      // and, when P > 1, keeps all of its rows' unit directions in LDS
  int Psh;            // log2(P)
};

// Device regions carved from the caller's workspace.  Per-sequence arrays are
// [BH][...] with sequence s = b*H + h outermost.  T (inputs, ring, outputs) is
// float or bf16 by Dims::bf16.  RT, the read-form storage type, is float on the
// fp32 path and fp16 on the bf16 path: every read-form quantity is bounded
// (LayerNorm output |k| <= sqrt(31), unit value direction |u| <= 1), so fp16
// keeps 3 more mantissa bits than bf16 at no range risk.
struct Dev {
  float* key_sum;    // [BH][S_cap][32] raw gated key sums (live dims)
  float* val_sum;    // [BH][S_cap][64] raw gated value sums
  int* count;        // [BH][S_cap]
  float* rho;        // [BH][S_cap] read radius
  void* unit;        // [BH][S_cap] x 128 B unit key direction: bf16 path [hi 32 | lo 32] bf16, fp32 path 32 f32
  void* kread;       // [BH][S_cap][32] RT current read-form key (live dims)
  void* vread;       // [BH][S_cap][64] T  current read-form value rho * u
  void* pkey;        // [BH][V_cap][32] RT read-form row versions: key
  void* pval;        // [BH][V_cap][64] T  read-form row versions: value rho * u
  float* prho;       // [BH][V_cap]       read-form row versions: radius
  int* pcount;       // [BH][V_cap]       read-form row versions: count
  float2* pnorm;     // [BH][V_cap]       read-form row versions: (LayerNorm 1/sqrt(var + eps), value scale)
  int* idx;          // [BH][idx_total] per absorbed chunk j: version id of each row after chunk j
  int* tslot;        // [BH][max_tokens] trace: row created / merged into
  uint8_t* tkind;    // [BH][max_tokens] trace: 0 sink 1 append 2 merge 255 none
  void* ring_k;      // [BH][R][64] T  rotated keys of the last R positions (slot = pos % R)
  void* ring_v;      // [BH][R][64] T
  float* ring_l;     // [BH][R] gate logits
  void* krot;        // [BH][max_tokens][32] bf16 rotated key dims [0, 32) (bf16, C >= 128; else null)
  float* rope_cos;   // [max_tokens][16]
  float* rope_sin;   // [max_tokens][16]
  int4* sched;       // [J_cap] (sinks_j, appends_j, rows_before_j, idx_off_j)
  int* nver;         // [BH] versions used
  uint2* xbuf;       // [BH][2][P][C] scan exchange: each workgroup's best per token (key bits, row | step tag)
  int* xerr;         // [1] set when a scan workgroup gave up waiting at an exchange
  int64_t* seq;      // [BH][kSeqFields] per-sequence launch parameters (sequences at their own positions)
};

// Per-sequence launch parameters (sequences at their own positions): a
// [BH][kSeqFields] int64 table; a kernel given one takes its sequence's entries
// in place of the launch-wide arguments.
enum SeqField {
  kSeqP0 = 0,   // first position of the call's inputs for this sequence
  kSeqJb,       // scan: chunks [jb, je) to absorb
  kSeqJe,
  kSeqCb,       // attention: first query chunk, number of query chunks, end position
  kSeqNq,
  kSeqEnd,
  kSeqN,        // tokens of the call for this sequence (prefill; rows past it are padding)
  kSeqFrom,     // ring refresh: positions [from, to)
  kSeqTo,
  kSeqPos,      // decode: the sequence's position
  kSeqActive,   // decode: 1 if the sequence takes a token in this step
  kSeqFields = 16
};

// Token source for a launch: positions >= p0 come from the call's inputs
// ([BH][n_call][64] rows, gate [BH][n_call]); positions < p0 from the ring.
// With `seq` set, p0 (and the other per-sequence values) come from the table.
struct Src {
  const void* q;
  const void* k;
  const void* v;
  const float* l;
  int64_t p0;
  int64_t n_call;
  const int64_t* seq = nullptr;
};

// The data-independent size schedule as the device computes it (integer schedules only:
// fixed, sqrt and saturating; the same rules as the host's).
struct SchedParams {
  int C;          // chunk
  int ns;         // sinks
  int sched;      // kvm_sched (FIXED, SQRT or SATURATING)
  int max_slots;
  int alpha;
  int J;          // chunks to describe
};

// Bytes of the library's static device scratch (one per GPU, for kvm_prefill_noalloc).
constexpr size_t kScratchBytes = (size_t)128 << 20;
// Device address of the static scratch on the current device (looked up once per device).
hipError_t scratch_address(void** out);
// Initialise a workspace carved from the scratch for one call: RoPE table, schedule table
// (computed on the device), and zeroed counters and exchange buffers (fill kernels, no memset).
hipError_t launch_noalloc_init(const Dims& m, const Dev& d, const SchedParams& sp, double rope_theta,
                               hipStream_t st);

// Backward pass: the forward's inputs, the output gradient, and where the input
// gradients go (all [BH][N][64] / [BH][N]; gradients float32).
struct BwdIn {
  const void* q;
  const void* k;
  const void* v;
  const float* l;
  const void* dout;
  int64_t N;         // tokens of the prefill being differentiated (positions [0, N))
};
// Backward buffers (carved from the caller's backward workspace) and outputs.
struct Bwd {
  float* part_win;     // [BH][nq][R][128]     per (query chunk, window key): dk (rotated) 64 | dv 64
  float* part_state;   // [BH][idx_total][96]  per (snapshot j, row): read-form gradient (key 32 | value 64),
                       //                      then the running totals of the row's sums after chunk j
  float* tot_rho;      // [BH][idx_total]      running total of the radius gradient
  float2* lse_d;       // [BH][N]              per query: log2 of the softmax denominator, D = sum P dP
  float* qr32;         // [BH][N][64]          rotated queries, fp32
  float* kr32;         // [BH][N][64]          rotated keys, fp32 (bf16 path: the same bytes as bf16 hi 64 | lo 64 per row)
  float* dq;           // [BH][N][64]
  float* dk;           // [BH][N][64]
  float* dv;           // [BH][N][64]
  float* dl;           // [BH][N]
  int nq;              // query chunks ceil(N / C)
  int absorbed;        // snapshots (absorbed chunks)
};
hipError_t launch_backward(const Dims& m, const Dev& d, const BwdIn& in, const Bwd& b, int rows_last,
                           hipStream_t st);

// Projections around the layer: C[m][n] = sum_k A[m][k] W[n][k].
struct ProjArgs {
  const void* x;      // in: x [M = B*N][K]; out: the layer output o [B*H][N][64]
  const void* w;      // [Nout][K]
  const float* bias;  // in: per-head gate-logit bias [H] or null
  void* q;            // in: [B*H][N][64]
  void* k;
  void* v;
  float* gl;          // in: gate logits [B*H][N]
  void* y;            // out: [M][Nout]
  int64_t M;          // B * N
  int64_t N;          // tokens per sequence
  int K;              // D = H * 64
  int Nout;           // in: 3D + H; out: D
  int H;
};
hipError_t launch_proj(const ProjArgs& a, bool out, bool is_bf16, hipStream_t st);

// Rows of unit directions a row-split scan workgroup keeps in LDS (bf16 path; 0 on the fp32 path).
int scan_lds_rows(int C, bool is_bf16);
hipError_t launch_init(const Dims& m, const Dev& d, double rope_theta, hipStream_t st);
// Absorb chunks [j_begin, j_end) for every sequence (sequential over j inside the kernel).
hipError_t launch_scan(const Dims& m, const Dev& d, const Src& src, int j_begin, int j_end, hipStream_t st);
// Attention for query chunks [c_begin, c_begin + n_q); queries at positions < end_pos; out rows
// are [BH][n_call][64] indexed by position - src.p0.  s_max: rows of the largest snapshot the
// chunks read.  With d.krot set, the rotated keys of the call must be in krot (launch_rope_keys).
hipError_t launch_attn(const Dims& m, const Dev& d, const Src& src, int64_t c_begin, int n_q, int64_t end_pos,
                       void* out, int s_max, hipStream_t st);
// Rotated key dims [0, 32) of the call's tokens into d.krot (no-op when d.krot is null).
hipError_t launch_rope_keys(const Dims& m, const Dev& d, const Src& src, hipStream_t st);
// Copy positions [from, to) of the call inputs into the ring (keys rotated).
hipError_t launch_ring_fill(const Dims& m, const Dev& d, const Src& src, int64_t from, int64_t to, hipStream_t st);
// Zero sequence s's version counter and exchange records, and (with the trace) mark its positions
// not absorbed: one sequence returned to an empty state.
hipError_t launch_seq_reset(const Dims& m, const Dev& d, int s, hipStream_t st);
// Decode step at position t: write token t (rotated key, value, gate logit) into ring
// slot t % R, then attend over `rows` state rows and the window; out [BH][64].
hipError_t launch_decode(const Dims& m, const Dev& d, const void* q, const void* k, const void* v, const float* l,
                         int64_t t, int rows, void* out, hipStream_t st, const int64_t* seq = nullptr);
// Gather the read form of snapshot j (rows_j rows, version list at idx_off) into
// key [BH][stride][32] RT, value rho * u [BH][stride][64] T, radius and count [BH][stride]
// (rows [0, rows) of each sequence; any output may be null; stride >= rows).
hipError_t launch_snapshot_gather(const Dims& m, const Dev& d, int rows, int64_t idx_off, int stride, void* key_out,
                                  void* val_out, float* rho_out, int* count_out, hipStream_t st);
// After the raw state (key_sum, val_sum, count, rho: `rows` rows per sequence) has been
// written into the workspace: derive every row's unit direction, current read form and a
// row version (version id = row, nver = rows), and the index list at idx_off of the last
// absorbed chunk (idx_off < 0: none).
hipError_t launch_state_load(const Dims& m, const Dev& d, int rows, int64_t idx_off, hipStream_t st);

}  // namespace kvm
