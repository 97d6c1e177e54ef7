// gfx950 (CDNA4) kernels of the Key-Value Means attention layer.
//
// Layer: [KVM abstract]; [KVM summary, Methodology; Core mechanisms 1-5].
//   scan_kernel     absorbs window-overflow chunks into the state: sinks,
//                   surprise top-m appends, winner-take-all cosine merge with
//                   a scalar gate into raw sums and counts, and emits a new
//                   read-form version of every row it touched.
//   attn_kernel     one softmax over [state read form || window] per query
//                   chunk, MFMA for Q.K^T and P.V, online softmax.
//   dec_*           single-token decode: ring write, split-K attention, combine.
//
// Wave64 throughout.  MFMA lane layouts used (checked on gfx950):
//   v_mfma_f32_32x32x16_bf16: A lane l holds A[l%32][8*(l/32)+e], B lane l holds
//     B[8*(l/32)+e][l%32] (e = 0..7); D lane l reg r is D[8*(r/4)+4*(l/32)+r%4][l%32].
//   v_mfma_f32_32x32x2f32: A lane l holds A[l%32][l/32], B lane l holds B[l/32][l%32];
//     D as above.
// Any consistent permutation of the contraction index between A and B is
// free; the kernels pick the one that makes each lane's loads contiguous.
#include <hip/hip_runtime.h>
#include <limits.h>
#include <type_traits>
#include <math.h>

#include "kvm.h"
#include "kvm_device.h"
#include "kvm_internal.h"

#include <algorithm>
#include <mutex>

// Device scratch for kvm_prefill_noalloc, the entry point for callers that
// cannot allocate device memory: the whole workspace of one call lives here
// (each GPU holds its own copy until the process ends).  Host code reaches it
// only through the address hipGetSymbolAddress gives (kvm::scratch_address).
static __device__ __align__(256) uint8_t scratch[kvm::kScratchBytes];
static_assert(kvm::kScratchBytes == KVM_NOALLOC_SCRATCH_BYTES, "scratch size as declared in kvm.h");

namespace kvm {
namespace {

// =====================================================================
// Initialisation: RoPE table in double precision, rounded to fp32.
// [KVM summary, Core mechanisms 4]: the window keeps RoPE.  Rotate-half
// pairing (j, j+16), frequency theta^(-j/16), angle = position * frequency.
// =====================================================================
__global__ void rope_table_kernel(float* cosv, float* sinv, int64_t max_tokens, double theta) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= max_tokens * 16) return;
  const int64_t pos = i >> 4;
  const int j = (int)(i & 15);
  const double f = pow(theta, -(double)j / 16.0);
  const double a = (double)pos * f;
  cosv[i] = (float)cos(a);
  sinv[i] = (float)sin(a);
}

// =====================================================================
// Scan: absorb overflowed chunks.
// [KVM summary, Core mechanisms 1]: a chunk that overflows the window updates
//   the state instead of being dropped.
// [KVM summary, Core mechanisms 2]: each overflowed key goes to the single
//   most similar state key (cosine), scaled by a data-dependent gate, into raw
//   sums and counts ([KVM lay summary, smart merge]).
// [KVM summary, Core mechanisms 3]: the least redundant overflowed tokens are
//   appended as new rows; the count m_j comes from the size schedule.
// [KVM summary, Core mechanisms 5]: the first tokens become protected sinks.
// One workgroup (8 waves) per sequence, or P of them sharing a sequence's
// rows (every P-th 32-row tile each; see scan_kernel), sequential over chunks.
// Per chunk:
//   1. the chunk's live keys, values and gates are in LDS (loaded into
//      registers during the previous step, stored at its end);
//   2. surprise: best cosine of every token against the non-sink rows that
//      existed before the chunk (MFMA over row tiles, next tile prefetched);
//      with P > 1 each workgroup takes its own rows and the P bests per token
//      are exchanged through memory;
//   3. append the m_j tokens of smallest (surprise, position) (parallel rank);
//   4. best cosine against the just-appended rows; assignment = better of the
//      two (lower row on ties);
//   5. the four lanes of the first token on each touched row (the creating
//      token for a new row) find the row's tokens by scanning the chunk's
//      targets, add them in position order (deterministic, no atomics) and
//      write the row's new read-form version (with P > 1, only for the rows
//      the workgroup owns; steps 3 and 4 run identically in every workgroup).
// Cosines: argmax over rows of cos(k, K_i) = argmax of dot(k, K_i/|K_i|).  On
// the bf16 path k is exact in bf16 and the unit direction U_i = K_i/|K_i| is
// split into bf16 hi + lo (|U - hi - lo| <= 2^-18 |U|), so two bf16 MFMA
// passes give dot(k, U_i) to ~1e-5 relative.  fp32 path: fp32 MFMA.
// =====================================================================
// Workgroup geometry per chunk size.  Eight waves: each holds CTW token blocks
// of 32 in the cosine pass (at most 4, for registers); TS wave groups split the
// chunk's tokens and the WG waves of a group stride over the state rows.  (12
// or 16 waves with the tokens split further measured slower: the cosine pass
// is MFMA/VALU-bound per SIMD, and splitting lengthens each wave's tile chain.)
template <int C>
struct ScanGeom {
  static constexpr int NW = 8;                        // waves
  static constexpr int NT = 64 * NW;                  // threads
  static constexpr int CT = C / 32;                   // token blocks of 32
  static constexpr int CTW = CT < 4 ? CT : 4;         // token blocks per wave
  static constexpr int TS = CT / CTW;                 // token groups
  static constexpr int WG = NW / TS;                  // waves sharing one token group (tile stride)
};

// Cosine-pass geometry of the row-split scan: a workgroup holds about a
// quarter of the rows or less, so waves take at most 2 token blocks and more
// waves share each token group's tiles (better balance over few tiles).
template <int C, bool PART>
struct CosGeom : ScanGeom<C> {};
template <int C>
struct CosGeom<C, true> : ScanGeom<C> {
  static constexpr int CTW = ScanGeom<C>::CT < 2 ? ScanGeom<C>::CT : 2;
  static constexpr int TS = ScanGeom<C>::CT / CTW;
  static constexpr int WG = ScanGeom<C>::NW / TS;
};

constexpr int pow2_floor(int x) { return x >= 2 ? 2 * pow2_floor(x / 2) : 1; }
constexpr int kSink = 0, kAppend = 1, kMerge = 2;

// Ranking geometry: P threads per token, each counting the smaller keys in
// one span of SPAN tokens.  Spans are stored SPAN + 4 words apart so that the
// P addresses one LDS cycle serves (one per span) fall in different banks.
template <int C>
struct RankGeom {
  static constexpr int NT = ScanGeom<C>::NT;
  static constexpr int P = pow2_floor(NT / C < C / 4 ? NT / C : C / 4);
  static constexpr int SPAN = C / P;
};
template <int C>
__device__ __forceinline__ int rank_slot(int t) {
  return t + 4 * (t / RankGeom<C>::SPAN);
}

// Chunk buffers: with NBUF = 2 the next chunk is stored into the spare buffer
// at the end of a step; with one buffer it is stored at the top of its own step.
template <typename T, int C>
struct ScanBuf {
  static constexpr int NBUF = C <= 128 ? 2 : 1;
};

constexpr int kVerCap = 4096;   // rows whose current version ids the scan keeps in LDS

template <typename T, int C>
struct ScanChunk {
  alignas(16) T k[C][32];   // live key dims of the chunk's tokens
  // bf16: the same scaled for the argmax keys (k 2^-e, |k| = m 2^e, m in [0.5, 1))
  alignas(16) T ks[Is<T>::bf ? C : 1][32];
  alignas(16) T v[C][64];   // values
  float g[C];               // merge gates
  float kn[C];              // |k live|
};

// PART: the row-split kernel, which keeps the version ids of its sink and own
// rows only (at most C + 512: the host splits only when a workgroup's rows
// fit its LDS cache of at most 512 rows), indexed by vslot.
template <typename T, int C, bool PART = false>
struct ScanSmem {
  static constexpr int RW = CosGeom<C, PART>::WG;   // waves whose bests the cosine pass combines
  static constexpr int VC = PART ? C + 512 : kVerCap;
  ScanChunk<T, C> ch[ScanBuf<T, C>::NBUF];
  alignas(16) uint32_t key[C + 4 * RankGeom<C>::P];   // sort keys (padded spans: rank_slot)
  float red_v[RW][C];
  int red_r[RW][C];
  float bE[C];
  int rE[C];
  int flag[C];
  int arow[C];        // row each token merges into or creates
  // row of each merged token (-1 for the others); the update scans the tokens
  // in four quarters, stored C/4 + 4 words apart so that the four quarters'
  // reads of one LDS cycle fall in different banks
  alignas(16) int mrow[C + 16];
  // the chunk's appended tokens: up to C = 128 one bit per position, beyond
  // that the list in position order (with per-wave counts to place them)
  alignas(16) uint32_t amask[C / 32];
  int app_list[C <= 128 ? 1 : C];
  int wtot[ScanGeom<C>::NW];
  int xok;                        // 0 after a wait at the exchange timed out
  int ver_cur[VC];                // current version id of every (own) row
  // row-split kernel up to C = 128: per own row (by version slot), the chunk's
  // tokens that merge into it, one bit per position
  static constexpr bool TAB = PART && C <= 128;
  static constexpr int MW = C / 32;
  alignas(16) uint32_t rmask[TAB ? VC : 1][TAB ? MW : 1];
};

// Polls of an exchange record before a scan workgroup gives up (each poll is a
// memory round trip, so a few seconds): the
// workgroups of a sequence are all resident unless other kernels hold the
// CUs, which they release; the limit only guarantees that every wave ends.
constexpr int kSpinLimit = 1 << 22;

// A chunk's live keys, values and gate logits in registers, between loads
// issued one chunk step ahead and the stores into an LDS buffer: thread tid
// holds the 16-byte pieces tid, tid + NT, ... of the keys and of the values
// (piece p = token p / KP (VP), part p % KP (VP)) and token tid's logit.
template <typename T, int C>
struct ChunkRegs {
  static constexpr int EL = 16 / sizeof(T);
  static constexpr int KP = 32 / EL, VP = 64 / EL;
  static constexpr int NT = ScanGeom<C>::NT;
  static constexpr int NK = (C * KP + NT - 1) / NT, NV = (C * VP + NT - 1) / NT;
  u32x4 k[NK], v[NV];
  float l;
};

template <typename T, int C>
__device__ __forceinline__ void chunk_load(ChunkRegs<T, C>& r, const Dims& m, const Src& src, int s, int64_t P0,
                                           const T* ring_k, const T* ring_v, const float* ring_l) {
  using R = ChunkRegs<T, C>;
  const int tid = threadIdx.x;
  // the chunk's first token: a row of the call's input, or a ring slot (the
  // chunk size divides the ring size, so a chunk never wraps the ring)
  const T *kb, *vb;
  const float* lb;
  if (P0 >= src.p0) {
    const size_t r0 = (size_t)s * src.n_call + (size_t)(P0 - src.p0);
    kb = reinterpret_cast<const T*>(src.k) + r0 * 64;
    vb = reinterpret_cast<const T*>(src.v) + r0 * 64;
    lb = src.l + r0;
  } else {
    const size_t r0 = (size_t)(P0 % m.R);
    kb = ring_k + r0 * 64;
    vb = ring_v + r0 * 64;
    lb = ring_l + r0;
  }
  // unconditional loads (indexes past the chunk repeat its last piece; the
  // stores skip them), so that no wait is needed until the stores
#pragma unroll
  for (int i = 0; i < R::NK; ++i) {
    const int p = min(tid + i * R::NT, C * R::KP - 1);
    r.k[i] = *reinterpret_cast<const u32x4*>(kb + (p / R::KP) * 64 + 32 + (p % R::KP) * R::EL);
  }
#pragma unroll
  for (int i = 0; i < R::NV; ++i) {
    const int p = min(tid + i * R::NT, C * R::VP - 1);
    r.v[i] = *reinterpret_cast<const u32x4*>(vb + (p / R::VP) * 64 + (p % R::VP) * R::EL);
  }
  r.l = lb[min(tid, C - 1)];
}

// Store a chunk held in registers into an LDS buffer, with each token's live
// key norm (sum of squares over the KP lanes holding its pieces) and merge
// gate (logistic sigmoid of the logit; 1 when the gate is removed).

template <typename T, int C>
__device__ __forceinline__ void chunk_store(const ChunkRegs<T, C>& r, ScanChunk<T, C>& dst, bool no_gate) {
  using R = ChunkRegs<T, C>;
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < R::NK; ++i) {
    const int p = tid + i * R::NT;
    if (p < C * R::KP) *reinterpret_cast<u32x4*>(&dst.k[0][0] + p * R::EL) = r.k[i];
    const T* x = reinterpret_cast<const T*>(&r.k[i]);
    float n2 = 0.f;
#pragma unroll
    for (int e = 0; e < R::EL; ++e) n2 = fmaf(tof(x[e]), tof(x[e]), n2);
    n2 = group_sum<R::KP>(n2);
    const float kn = __builtin_amdgcn_sqrtf(n2);   // hardware square root (1 ulp)
    if constexpr (Is<T>::bf) {
      // k 2^-e, exact: each bf16 widened to fp32 (its bits in the upper half),
      // scaled, and narrowed back by taking the upper half
      int e;
      (void)frexpf(kn, &e);
      u32x4 ys;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t xw = r.k[i][q];
        const uint32_t lo = __float_as_uint(ldexpf(__uint_as_float(xw << 16), -e));
        const uint32_t hi = __float_as_uint(ldexpf(__uint_as_float(xw & 0xFFFF0000u), -e));
        ys[q] = (lo >> 16) | (hi & 0xFFFF0000u);
      }
      if (p < C * R::KP) *reinterpret_cast<u32x4*>(&dst.ks[0][0] + p * R::EL) = ys;
    }
    if (p < C * R::KP && p % R::KP == 0) dst.kn[p / R::KP] = kn;
  }
#pragma unroll
  for (int i = 0; i < R::NV; ++i) {
    const int p = tid + i * R::NT;
    if (p < C * R::VP) *reinterpret_cast<u32x4*>(&dst.v[0][0] + p * R::EL) = r.v[i];
  }
  // Every thread settles its gate-logit load here, also those whose value is
  // not stored: a load left pending would make a later reuse of its register
  // wait for all outstanding memory operations of the wave.
  float lg = r.l;
  asm volatile("" : "+v"(lg));
  // (hardware 2^x and reciprocal, each within 1 ulp)
  if (tid < C) dst.g[tid] = no_gate ? 1.0f : __builtin_amdgcn_rcpf(1.0f + exp2_fast(-lg * kLog2e));
}

// One lane's quarter of the row a merged token goes to: key dims [8 sub,
// 8 sub + 8), value dims [16 sub, 16 sub + 16), count and radius.  Loaded once
// the chunk's assignment is known, consumed by the update.
struct RowRegs {
  f32x4 k[2], v[4];
  int n;
  float rh;
};

__device__ __forceinline__ void row_load(RowRegs& r, const float* key_sum, const float* val_sum, const int* count,
                                         const float* rho, int row, int sub) {
  const f32x4* ks = reinterpret_cast<const f32x4*>(key_sum + (size_t)row * 32 + 8 * sub);
  const f32x4* vs = reinterpret_cast<const f32x4*>(val_sum + (size_t)row * 64 + 16 * sub);
  r.k[0] = ks[0];
  r.k[1] = ks[1];
#pragma unroll
  for (int i = 0; i < 4; ++i) r.v[i] = vs[i];
  r.n = count[row];
  r.rh = rho[row];
}

// Argmax keys.  The surprise pass scales each token's live key by a power of
// two, 2^-e with |k| = m 2^e, m in [0.5, 1) (an exact scaling that does not
// change which row is most similar), and starts every accumulator at 2, so a
// tile holds 2 + dot(k', U_i) in (1, 3): positive floats, ordered like their
// bit patterns.  A value's key is its bit pattern with the 4 low mantissa bits
// replaced by 15 - r, r the lane's slot of the row (increasing with the row):
// one unsigned max over a lane's 16 slots gives the largest value to 2^-18
// (the split of U into bf16 halves is good to 2^-18 as well) and, among
// values equal at that precision, the lowest row.
constexpr float kKeyBase = 2.0f;

__device__ __forceinline__ float key_scale(float kn, int& e) {
  (void)frexpf(kn, &e);
  return ldexpf(1.0f, -e);
}

// Fold one 32x32 result tile into a lane's running best (truncated key bk, row
// br): the lane holds rows row0h + 8(r/4) + r%4 of its token (row0h = first
// row of the tile + 4h).  Tiles come in increasing row order and only a
// strictly larger truncated key replaces the best, so ties keep the lower row.
__device__ __forceinline__ void lane_best(const f32x16& acc, int row0h, uint32_t& bk, int& br) {
  uint32_t k[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) k[r] = (__float_as_uint(acc[r]) & ~0xFu) | (uint32_t)(15 - r);
  uint32_t m = max(max(k[0], k[1]), k[2]);
#pragma unroll
  for (int r = 3; r < 15; r += 2) m = max(max(m, k[r]), k[r + 1]);
  m = max(m, k[15]);
  const int r = 15 - (int)(m & 15u);
  const uint32_t mt = m & ~0xFu;
  const bool imp = mt > bk;
  br = imp ? row0h + r + (r & 12) : br;
  bk = imp ? mt : bk;
}

// Everything derived from one state row's raw sums, computed by the row's
// group of four lanes (lane sub owns key dims [8 sub, 8 sub + 8) and value
// dims [16 sub, 16 sub + 16)): the unit key direction K/|K| for the cosine
// passes (bf16 path: bf16 hi + lo halves; also into the LDS copy `ulrow` when
// not null) and the just-in-time read form ([KVM summary, Core mechanisms 2]):
// LayerNorm of K/n over the live dims (no affine) and the value rho * V/|V|
// (direction of the sum at the radius fixed at creation; the plain mean V/n
// without value-length normalisation), written as the current read form and
// as a row version.  The absorption scan and the state load share this code,
// so a loaded state reads back bit for bit like the one it was exported from.
template <typename T>
__device__ __forceinline__ void row_derive(const float (&K)[8], const float (&V)[16], int n, float rh, int sub,
                                           const Dims& m, char* unit_row, bf16* ulrow,
                                           typename Rd<T>::type* kread_row, T* vread_row,
                                           typename Rd<T>::type* pkey_ver, T* pval_ver, float& rs_out,
                                           float& vsc_out) {
  using RT = typename Rd<T>::type;
  constexpr int REL = 16 / sizeof(RT);
  // row sums of squares and moments over the four lanes
  float k2 = 0.f, ksum = 0.f, v2 = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) { k2 = fmaf(K[i], K[i], k2); ksum += K[i]; }
#pragma unroll
  for (int i = 0; i < 16; ++i) v2 = fmaf(V[i], V[i], v2);
  k2 = quad_sum(k2);
  ksum = quad_sum(ksum);
  v2 = quad_sum(v2);
  {
    const float inv = k2 > 0.f ? __builtin_amdgcn_rsqf(k2) : 0.f;   // 1 ulp
    if constexpr (Is<T>::bf) {
      alignas(16) bf16 hi[8], lo[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float y = K[i] * inv;
        hi[i] = (bf16)y;
        lo[i] = (bf16)(y - (float)hi[i]);
      }
      copy16(unit_row + 16 * sub, hi);
      copy16(unit_row + 64 + 16 * sub, lo);
      if (ulrow) {
        copy16(ulrow + 8 * sub, hi);
        copy16(ulrow + 32 + 8 * sub, lo);
      }
    } else {
      alignas(16) float uu[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) uu[i] = K[i] * inv;
      copy16(unit_row + 32 * sub, uu);
      copy16(unit_row + 32 * sub + 16, uu + 4);
    }
  }
  const float invn = __builtin_amdgcn_rcpf((float)n);   // 1 ulp
  const float mean = ksum * invn * (1.0f / 32.0f);
  float var = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) { const float dx = K[i] * invn - mean; var = fmaf(dx, dx, var); }
  var = quad_sum(var);
  var *= (1.0f / 32.0f);
  const float rs = __builtin_amdgcn_rsqf(var + m.ln_eps);
  const float vsc = m.no_vnorm ? invn : (v2 > 0.f ? rh * __builtin_amdgcn_rsqf(v2) : 0.f);
  rs_out = rs;
  vsc_out = vsc;
  alignas(16) RT kh[8];
  alignas(16) T vh[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) kh[i] = fromf<RT>((K[i] * invn - mean) * rs);
#pragma unroll
  for (int i = 0; i < 16; ++i) vh[i] = fromf<T>(V[i] * vsc);
#pragma unroll
  for (int i = 0; i < 8; i += REL) {
    copy16(pkey_ver + 8 * sub + i, &kh[i]);
    copy16(kread_row + 8 * sub + i, &kh[i]);
  }
#pragma unroll
  for (int i = 0; i < 16; i += REL) {
    copy16(pval_ver + 16 * sub + i, &vh[i]);
    copy16(vread_row + 16 * sub + i, &vh[i]);
  }
}

// bf16 path: one 32-row tile of unit directions (hi and lo halves) as the MFMA
// A operand: lane (jl, h) holds dims [16h, 16h+16) of row rb + 32 tile + jl.
// The first NL rows the pass reads (from row LB: 0, or the first row after the
// protected sinks) are also kept in LDS, hi and lo halves in a row of UL_PITCH
// elements (padded so that 16 lanes reading 16 rows hit distinct banks); the
// update writes both copies.
// Rows past re - 1 repeat row re - 1: equal values at higher rows, which never
// win a tie, so they need no mask.
struct UnitTiles {
  bf16x8 a0[4], a1[4];
};
constexpr int UL_PITCH = 72;
template <typename T, int C, bool PART = false>
struct ScanUnitLds {
  static constexpr int avail = 163840 - (int)sizeof(ScanSmem<T, C, PART>) - 512;
  static constexpr int fit = avail / (UL_PITCH * 2);
  static constexpr int NL = !Is<T>::bf ? 0 : (fit >= 512 ? 512 : (fit > 0 ? fit & ~31 : 0));   // rows
};
// Row partition: a sequence's rows from LB on are split into 32-row tiles,
// and of P = 2^psh workgroups, workgroup p owns tiles p, p + P, ... (rows
// below LB, the protected sinks, belong to workgroup 0).  A workgroup numbers
// its own tiles locally (k = 0, 1, ...: global tile p + k P).
__device__ __forceinline__ int own_tiles(int ntile, int p, int psh) {
  return ntile > p ? ((ntile - 1 - p) >> psh) + 1 : 0;
}
// LDS slot of own row r >= LB: local tile * 32 + offset in the tile
__device__ __forceinline__ int own_slot(int r, int LB, int psh) {
  return ((((r - LB) >> 5) >> psh) << 5) + ((r - LB) & 31);
}
// LDS-resident local tiles of rows [rb, re) (rb == LB): the first NL / 32 of
// the workgroup's own tiles.
__device__ __forceinline__ int lds_tiles(int rb, int re, int LB, int NL, int p, int psh) {
  if (rb != LB || re <= rb) return 0;
  return min(own_tiles((re - rb + 31) >> 5, p, psh), NL >> 5);
}
// Global tile gt (own, local tile kt) from LDS; rows past re - 1 repeat row
// re - 1, which lies in the same (last) tile.
__device__ __forceinline__ void unit_tile_lds(const bf16* ul, int rb, int re, int LB, int gt, int psh,
                                              bf16x8 (&a)[4]) {
  const int lane = threadIdx.x & 63, jl = lane & 31, h = lane >> 5;
  const int ri = own_slot(min(rb + (gt << 5) + jl, re - 1), LB, psh);
  // (a 24-bit product: a 32-bit multiply-add is emitted as a 64-bit one whose
  // unused high addend half can be a register still being loaded)
  const bf16* u = ul + __umul24((unsigned)ri, (unsigned)UL_PITCH) + 16 * h;
  a[0] = *reinterpret_cast<const bf16x8*>(u);
  a[1] = *reinterpret_cast<const bf16x8*>(u + 8);
  a[2] = *reinterpret_cast<const bf16x8*>(u + 32);
  a[3] = *reinterpret_cast<const bf16x8*>(u + 40);
}
__device__ __forceinline__ void unit_tile_load(const char* unit, int rb, int re, int tile, bf16x8 (&a)[4]) {
  const int lane = threadIdx.x & 63, jl = lane & 31, h = lane >> 5;
  const int ri = min(rb + (tile << 5) + jl, re - 1);
  const bf16* u = reinterpret_cast<const bf16*>(unit) + (size_t)ri * 64 + 16 * h;
  a[0] = *reinterpret_cast<const bf16x8*>(u);
  a[1] = *reinterpret_cast<const bf16x8*>(u + 8);
  a[2] = *reinterpret_cast<const bf16x8*>(u + 32);
  a[3] = *reinterpret_cast<const bf16x8*>(u + 40);
}
// First local tile of this wave's share (wt, wt + WG, ...) that is not LDS-resident.
template <int C>
__device__ __forceinline__ int first_global_tile(int wt, int ntl) {
  constexpr int WG = ScanGeom<C>::WG;
  return wt >= ntl ? wt : wt + WG * ((ntl - wt + WG - 1) / WG);
}
// The first two global-memory tiles of this wave's share of the workgroup's
// rows in [rb, re) for cos_best, loaded ahead so that their latency overlaps
// the work before them.
template <int C>
__device__ __forceinline__ void cos_preload(const char* unit, int rb, int re, int ntl, int p, int psh,
                                            UnitTiles& pre) {
  using G = ScanGeom<C>;
  const int wt = (threadIdx.x >> 6) / G::TS;
  const int nown = own_tiles(re > rb ? (re - rb + 31) >> 5 : 0, p, psh);
  const int g0 = first_global_tile<C>(wt, ntl);
  if (g0 < nown) unit_tile_load(unit, rb, re, p + (g0 << psh), pre.a0);
  if (g0 + G::WG < nown) unit_tile_load(unit, rb, re, p + ((g0 + G::WG) << psh), pre.a1);
}

// Best (largest) dot(k_t, U_i) over this workgroup's rows i in [rb, re) for
// every token t of the chunk, compared on the argmax keys (to 2^-17 |k_t|);
// ties to the lowest row.  Hands the best key (as a float in (1, 3), 0 if
// the workgroup has no row) and its row (INT_MAX if none) of token t to
// emit(t, key, row), one thread per token, with no barrier after it;
// every thread calls settle() between its tile loop and the combine.
// All threads of the block must call it; on the bf16 path `pre` holds the
// tiles cos_preload fetched for the same rows.  PART: the rows are split over
// several workgroups and every own row is LDS-resident (ntl == own tiles).
template <typename T, int C, bool PART, typename Settle, typename Emit>
__device__ __forceinline__ void cos_best(ScanSmem<T, C, PART>& sm, const ScanChunk<T, C>& ch, const char* unit,
                                         const bf16* ul, int LB, int ntl, int rb, int re, int p, int psh,
                                         UnitTiles& pre, Settle&& settle, Emit&& emit) {
  using G = CosGeom<C, PART>;
  constexpr int CT = G::CTW;   // token blocks of this wave
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, jl = lane & 31, h = lane >> 5;
  const int tg = w % G::TS, wt = w / G::TS;   // token group, tile lane
  const int tok0 = 32 * CT * tg;              // first token of the group
  uint32_t bk[CT];
  int br[CT];
#pragma unroll
  for (int tt = 0; tt < CT; ++tt) { bk[tt] = 0u; br[tt] = INT_MAX; }
  const int nown = own_tiles(re > rb ? (re - rb + 31) >> 5 : 0, p, psh);   // own tiles (local k < nown)
  if (wt < nown) {
    // every accumulator starts at the key base (an inline constant of the MFMA)
    const f32x16 base = {kKeyBase, kKeyBase, kKeyBase, kKeyBase, kKeyBase, kKeyBase, kKeyBase, kKeyBase,
                         kKeyBase, kKeyBase, kKeyBase, kKeyBase, kKeyBase, kKeyBase, kKeyBase, kKeyBase};
    if constexpr (Is<T>::bf) {
      // lane half h owns dims [16h, 16h+16) of every 32-dim (scaled) key
      bf16x8 bfr[CT][2];
#pragma unroll
      for (int tt = 0; tt < CT; ++tt)
#pragma unroll
        for (int q = 0; q < 2; ++q)
          bfr[tt][q] = *reinterpret_cast<const bf16x8*>(&ch.ks[tok0 + 32 * tt + jl][16 * h + 8 * q]);
      auto load = [&](int kt, bf16x8 (&a)[4]) { unit_tile_load(unit, rb, re, p + (kt << psh), a); };
      auto tile_best = [&](const bf16x8 (&a)[4], int kt) {
        const int row0h = rb + ((p + (kt << psh)) << 5) + 4 * h;
        f32x16 acc[CT];
        // independent accumulators interleaved so dependent MFMAs are CT apart
#pragma unroll
        for (int tt = 0; tt < CT; ++tt) acc[tt] = mfma_bf16(a[0], bfr[tt][0], base);
#pragma unroll
        for (int tt = 0; tt < CT; ++tt) acc[tt] = mfma_bf16(a[1], bfr[tt][1], acc[tt]);
#pragma unroll
        for (int tt = 0; tt < CT; ++tt) acc[tt] = mfma_bf16(a[2], bfr[tt][0], acc[tt]);
#pragma unroll
        for (int tt = 0; tt < CT; ++tt) acc[tt] = mfma_bf16(a[3], bfr[tt][1], acc[tt]);
#pragma unroll
        for (int tt = 0; tt < CT; ++tt) lane_best(acc[tt], row0h, bk[tt], br[tt]);
      };
      // two register sets in ping-pong: the loads of tile i+2W are issued right
      // after the MFMAs of tile i read their set, so they overlap tile i+W
      constexpr int WG = G::WG;
      // LDS-resident tiles first (lowest rows), then the global ones.  Up to
      // C = 128 the next tile's fragments are read while this tile's products
      // run (two register sets; a read past the last tile re-reads the last one).
      if (C > 128) {   // (registers: one set)
        for (int kt = wt; kt < ntl; kt += WG) {
          bf16x8 b[4];
          unit_tile_lds(ul, rb, re, LB, p + (kt << psh), psh, b);
          tile_best(b, kt);
        }
      } else if (wt < ntl) {
        bf16x8 b0[4], b1[4];
        unit_tile_lds(ul, rb, re, LB, p + (wt << psh), psh, b0);
        for (int kt = wt; kt < ntl; kt += 2 * WG) {
          const int k1 = kt + WG;
          unit_tile_lds(ul, rb, re, LB, p + (min(k1, ntl - 1) << psh), psh, b1);
          tile_best(b0, kt);
          if (k1 >= ntl) break;
          unit_tile_lds(ul, rb, re, LB, p + (min(k1 + WG, ntl - 1) << psh), psh, b0);
          tile_best(b1, k1);
        }
      }
      if constexpr (!PART) {
        bf16x8(&a0)[4] = pre.a0;
        bf16x8(&a1)[4] = pre.a1;
        for (int kt = first_global_tile<C>(wt, ntl); kt < nown; kt += 2 * WG) {
          tile_best(a0, kt);
          if (kt + 2 * WG < nown) load(kt + 2 * WG, a0);
          if (kt + WG < nown) {
            tile_best(a1, kt + WG);
            if (kt + 3 * WG < nown) load(kt + 3 * WG, a1);
          }
        }
      }
    } else {
      // fp32: step kk contracts dims kk and 16+kk (lane half h holds dim 16h+kk)
      float bfr[CT][16];
#pragma unroll
      for (int tt = 0; tt < CT; ++tt)
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {
          int e;
          bfr[tt][kk] = tof(ch.k[tok0 + 32 * tt + jl][16 * h + kk]) * key_scale(ch.kn[tok0 + 32 * tt + jl], e);
        }
      const float* U = reinterpret_cast<const float*>(unit);
      for (int kt = wt; kt < nown; kt += G::WG) {
        const int row0 = rb + ((p + (kt << psh)) << 5);
        const int ri = min(row0 + jl, re - 1);
        const float* u = U + (size_t)ri * 32 + 16 * h;
        float a[16];
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) a[kk] = u[kk];
#pragma unroll
        for (int tt = 0; tt < CT; ++tt) {
          f32x16 acc = base;
#pragma unroll
          for (int kk = 0; kk < 16; ++kk) acc = mfma_f32(a[kk], bfr[tt][kk], acc);
          lane_best(acc, row0 + 4 * h, bk[tt], br[tt]);
        }
      }
    }
  }
  settle();
  // combine the two lane halves and the waves on (truncated key, row): the
  // larger key, or the lower row on equal keys
#pragma unroll
  for (int tt = 0; tt < CT; ++tt) {
    const uint32_t ok = partner_u32(bk[tt]);
    const int orow = partner_i(br[tt]);
    if (ok > bk[tt] || (ok == bk[tt] && orow < br[tt])) { bk[tt] = ok; br[tt] = orow; }
    if (h == 0 && wt < nown) {
      sm.red_v[wt][tok0 + 32 * tt + jl] = __uint_as_float(bk[tt]);
      sm.red_r[wt][tok0 + 32 * tt + jl] = br[tt];
    }
  }
  lds_barrier();
  const int nw = min(nown, G::WG);
  for (int t = tid; t < C; t += G::NT) {
    if constexpr (G::WG < 4) {   // two waves: a short loop (and fewer live registers)
      float v = 0.f;
      int r = INT_MAX;
      for (int ww = 0; ww < nw; ++ww) {
        const float ov = sm.red_v[ww][t];
        const int orow = sm.red_r[ww][t];
        if (ov > v || (ov == v && orow < r)) { v = ov; r = orow; }
      }
      emit(t, v, r);
      continue;
    }
    // every wave's partial is read first (independent LDS reads in flight
    // together), then combined; slots of waves without tiles are skipped
    float pv[G::WG];
    int pr[G::WG];
#pragma unroll
    for (int ww = 0; ww < G::WG; ++ww) {
      pv[ww] = sm.red_v[ww][t];
      pr[ww] = sm.red_r[ww][t];
    }
    float v = 0.f;
    int r = INT_MAX;
#pragma unroll
    for (int ww = 0; ww < G::WG; ++ww)
      if (ww < nw && (pv[ww] > v || (pv[ww] == v && pr[ww] < r))) { v = pv[ww]; r = pr[ww]; }
    emit(t, v, r);
  }
}

// Position of the k-th set bit (k from 0) of the NW-word mask m (it has more
// than k set bits): the word by running popcounts, then the bit by halving.
template <int NW>
__device__ __forceinline__ int kth_bit(const uint32_t (&m)[NW], int k) {
  uint32_t x = m[0];
  int base = 0;
#pragma unroll
  for (int i = 0; i + 1 < NW; ++i) {
    const int c = __popc(x);
    const bool on = k >= c && base == 32 * i;   // still past word i
    k = on ? k - c : k;
    x = on ? m[i + 1] : x;
    base = on ? 32 * (i + 1) : base;
  }
  int bit = 0;
#pragma unroll
  for (int w = 16; w >= 1; w >>= 1) {
    const int c = __popc(x & ((1u << w) - 1u));
    const bool up = k >= c;
    k = up ? k - c : k;
    x = up ? x >> w : x;
    bit = up ? bit + w : bit;
  }
  return base + bit;
}

// rank[t] = #{s : key[s] < key[t]} for every t < C (tokens to leave out carry
// the largest key), using up to all threads: P = min(threads / C, C / 4) lanes
// per token, each over C / P keys read four at a time, summed across the P
// lanes.  Returns the rank on the lane with part == 0 (else -1) and that
// lane's token in t_out.
template <int C>
__device__ __forceinline__ int parallel_rank(const uint32_t* key, int& t_out) {
  using G = RankGeom<C>;
  constexpr int P = G::P, SPAN = G::SPAN;
  static_assert(SPAN % 4 == 0, "keys are read in fours");
  const int t = threadIdx.x / P, part = threadIdx.x % P;
  t_out = t;
  int cnt = 0;
  if (t < C) {
    const uint32_t kt = key[rank_slot<C>(t)];
    const u32x4* kp = reinterpret_cast<const u32x4*>(key + part * (SPAN + 4));
#pragma unroll
    for (int i = 0; i < SPAN / 4; ++i) {
      const u32x4 k4 = kp[i];
      cnt += (k4[0] < kt) + (k4[1] < kt) + (k4[2] < kt) + (k4[3] < kt);
    }
  }
  cnt = group_sum<P>(cnt);
  return (t < C && part == 0) ? cnt : -1;
}

// PART: the sequence's rows are split over P = 2^Psh > 1 workgroups, each
// holding all of its own rows' unit directions in LDS (the host picks P so
// that they fit), with one exchange of per-token bests per chunk; otherwise
// one workgroup per sequence, rows past the LDS-resident ones streamed from
// global memory.
template <typename T, int C, bool PART>
__global__ __launch_bounds__(ScanGeom<C>::NT) void scan_kernel(Dims m, Dev d, Src src, const int4* __restrict__ sched,
                                                                 int j_begin, int j_end) {
  constexpr int kScanThreads = ScanGeom<C>::NT;
  constexpr int kScanWaves = ScanGeom<C>::NW;
  using RT = typename Rd<T>::type;
  constexpr int REL = 16 / sizeof(RT);     // read-form elements per 16-byte piece
  constexpr int NBUF = ScanBuf<T, C>::NBUF;
  constexpr int TP = (4 * C + kScanThreads - 1) / kScanThreads;   // token groups of four lanes per thread
  __shared__ ScanSmem<T, C, PART> sm;
  constexpr int NL = ScanUnitLds<T, C, PART>::NL;
  __shared__ alignas(16) bf16 ul[NL > 0 ? NL : 1][UL_PITCH];
  // Workgroup p of the P = 2^psh that share sequence s (each owns every P-th
  // 32-row tile of the rows from LB on).  With the sequence count a multiple
  // of 8, a sequence's workgroups are P consecutive dispatches on one XCD
  // (dispatch b goes to XCD b mod 8), so their exchanges stay in one L2.
  const int psh = PART ? m.Psh : 0;
  int s, p;
  if constexpr (PART) {
    const int b = blockIdx.x;
    if (m.BH % 8 == 0) {
      const int k = b >> 3;
      s = ((k >> psh) << 3) + (b & 7);
      p = k & (m.P - 1);
    } else {
      s = b >> psh;
      p = b & (m.P - 1);
    }
  } else {
    s = blockIdx.x;
    p = 0;
  }
  if (src.seq) {   // this sequence's own chunk range and input position
    const int64_t* sr = src.seq + (size_t)s * kSeqFields;
    src.p0 = sr[kSeqP0];
    j_begin = (int)sr[kSeqJb];
    j_end = (int)sr[kSeqJe];
  }
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int LB = m.unprot ? 0 : m.ns;   // first row of the tile partition
  auto own = [&](int r) {
    if constexpr (PART) return r < LB ? p == 0 : (((r - LB) >> 5) & (m.P - 1)) == p;
    else return true;
  };
  // slot of an own row's current version id in LDS
  auto vslot = [&](int r) {
    if constexpr (PART) return r < LB ? r : LB + own_slot(r, LB, psh);
    else return r;
  };
  // f(slot, row) for every own row below `rows`, one thread per LDS slot (the
  // sink rows, then the own tiles' rows in slot order), over the first `nthr`
  // threads
  auto for_own_rows = [&](int rows, auto&& f, int nthr = ScanGeom<C>::NT) {
    if constexpr (PART) {
      const int nt = own_tiles(rows > LB ? (rows - LB + 31) >> 5 : 0, p, psh);
      for (int q = tid; q < LB + 32 * nt; q += nthr) {
        if (q < LB) {
          if (p == 0 && q < rows) f(q, q);
        } else {
          const int ls = q - LB;
          const int r = LB + ((p + ((ls >> 5) << psh)) << 5) + (ls & 31);
          if (r < rows) f(q, r);
        }
      }
    } else {
      for (int i = tid; i < rows; i += nthr) f(i, i);
    }
  };

  float* key_sum = d.key_sum + (size_t)s * m.S_cap * 32;
  float* val_sum = d.val_sum + (size_t)s * m.S_cap * 64;
  int* count = d.count + (size_t)s * m.S_cap;
  float* rho = d.rho + (size_t)s * m.S_cap;
  char* unit = reinterpret_cast<char*>(d.unit) + (size_t)s * m.S_cap * 128;
  RT* kread = reinterpret_cast<RT*>(d.kread) + (size_t)s * m.S_cap * 32;
  T* vread = reinterpret_cast<T*>(d.vread) + (size_t)s * m.S_cap * 64;
  RT* pkey = reinterpret_cast<RT*>(d.pkey) + (size_t)s * m.V_cap * 32;
  T* pval = reinterpret_cast<T*>(d.pval) + (size_t)s * m.V_cap * 64;
  float* prho = d.prho + (size_t)s * m.V_cap;
  int* pcount = d.pcount + (size_t)s * m.V_cap;
  int* idx = d.idx + (size_t)s * m.idx_total;
  const T* ring_k = reinterpret_cast<const T*>(d.ring_k) + (size_t)s * m.R * 64;
  const T* ring_v = reinterpret_cast<const T*>(d.ring_v) + (size_t)s * m.R * 64;
  const float* ring_l = d.ring_l + (size_t)s * m.R;
  int nver = d.nver[s];
  // the current version of every row lives in LDS; each chunk's index list is
  // written out from it at the start of the next step (stores only)
  const bool ver_lds = PART || m.S_cap <= kVerCap;
  if (ver_lds && j_begin > 0 && j_begin < j_end) {
    const int r0 = sched[j_begin].z;
    const int* prev = idx + sched[j_begin - 1].w;
    for_own_rows(r0, [&](int q, int r) { sm.ver_cur[q] = prev[r]; });
  }

  constexpr bool kTab = ScanSmem<T, C, PART>::TAB;
  constexpr int MW = ScanSmem<T, C, PART>::MW;
  if constexpr (kTab)
    for (int i = tid; i < ScanSmem<T, C, PART>::VC * MW; i += kScanThreads) (&sm.rmask[0][0])[i] = 0u;
  int clear_slot = -1;   // a mask this thread's lane group read, cleared in the next step
  if (tid < C / 32) sm.amask[tid] = 0u;

  // unit directions kept in LDS: the first NL rows of the workgroup's own
  // tiles (local slot = local tile * 32 + offset) that exist at the start
  if (NL > 0 && j_begin < j_end) {
    const int R0s = sched[j_begin].z;
    const int nfill = min(own_tiles(R0s > LB ? (R0s - LB + 31) >> 5 : 0, p, psh) * 32, NL);
    for (int q = tid; q < nfill * 8; q += kScanThreads) {
      const int ls = q >> 3;
      const int r = LB + ((p + ((ls >> 5) << psh)) << 5) + (ls & 31);
      if (r < R0s) copy16(&ul[ls][(q & 3) * 8 + ((q >> 2) & 1) * 32], unit + (size_t)r * 128 + 16 * (q & 7));
    }
  }

  // the chunk in flight: loaded one step ahead, stored into LDS at the end of
  // the step before its own (two buffers) or at the top of its own step (one)
  ChunkRegs<T, C> cr;
  if (j_begin < j_end) {
    chunk_load<T, C>(cr, m, src, s, (int64_t)j_begin * C, ring_k, ring_v, ring_l);
    if constexpr (NBUF == 2) {
      chunk_store<T, C>(cr, sm.ch[0], m.no_gate);
      __syncthreads();
    }
  }

  // Within a chunk step threads exchange data through LDS only (LDS barriers,
  // so loads stay in flight); every global write of a step is read by another
  // thread only in a later step, after the barrier that closes the step.
  // Row-split kernel with two chunk buffers: the next chunk loads during the
  // surprise pass (which reads LDS only) and is stored into the spare buffer
  // while the exchange records travel, off the step's critical path.
  constexpr bool kEarly = PART && NBUF == 2;
  int4 sc_next = j_begin < j_end ? sched[j_begin] : make_int4(0, 0, 0, 0);
  int prev_off = j_begin > 0 ? sched[j_begin - 1].w : 0;
  int last_rows = 0;
  for (int j = j_begin; j < j_end; ++j) {
    const int cur = NBUF == 2 ? (j - j_begin) & 1 : 0;
    ScanChunk<T, C>& chc = sm.ch[cur];
    const int4 sc = sc_next;
    const int sinks = sc.x, mj = sc.y, R0 = sc.z;
    const int64_t ioff = sc.w;
    const int nc = sinks + mj;
    const int rows_after = R0 + nc;
    const int64_t P0 = (int64_t)j * C;

    // the token masks of the rows the previous step updated (every read of
    // them came before the barrier that closed that step)
    if constexpr (kTab)
      if (clear_slot >= 0) {
        if ((tid & 3) == 0)
          for (int i = 0; i < MW; ++i) sm.rmask[clear_slot][i] = 0u;
        clear_slot = -1;
      }
    // ---- 1. the chunk, its key norms and gates are in LDS buffer `cur` (one
    // buffer: store it now); the first unit-direction tiles of the surprise
    // pass start loading.  The next chunk's loads are issued before the index
    // list's stores below, so that they do not queue behind them.
    if constexpr (NBUF == 1) {
      chunk_store<T, C>(cr, chc, m.no_gate);
      lds_barrier();
    }
    if constexpr (kEarly)
      if (j + 1 < j_end) chunk_load<T, C>(cr, m, src, s, P0 + C, ring_k, ring_v, ring_l);
    // index list of the previous step (its rows are the R0 rows before this chunk);
    // the row-split kernel writes it at the end of its surprise pass
    if (!PART && ver_lds && j > j_begin) for_own_rows(R0, [&](int q, int r) { idx[prev_off + r] = sm.ver_cur[q]; });
    // surprise is measured against the non-sink rows that existed before the
    // chunk (every row before the chunk when sinks are unprotected)
    const int eb = m.unprot ? 0 : min(m.ns, R0), ee = R0;
    UnitTiles pre;
    const int ntl = NL > 0 ? lds_tiles(eb, ee, LB, NL, p, psh) : 0;
    if constexpr (Is<T>::bf && !PART) cos_preload<C>(unit, eb, ee, ntl, p, psh, pre);
    const T (*Kc)[32] = chc.k;
    const T (*Vc)[64] = chc.v;
    // token t's best over the rows before the chunk, from its argmax key v
    // (row r): back to the dot product (subtract the key base, exact on
    // (1, 3), and undo the token's power-of-two scaling), and its ranking key
    // = (surprise to 2^-15, position): smaller = more surprising; sinks never
    // rank.  (The low 8 bits of the ordered surprise give way to the position,
    // C <= 256; surprises that close are a near tie.)
    auto token_key = [&](int t, float v, int r) {
      int e;
      (void)key_scale(chc.kn[t], e);
      const float be = r == INT_MAX ? -kInf : ldexpf(v - kKeyBase, e);
      sm.bE[t] = be;
      sm.rE[t] = r;
      float mu;
      if (ee > eb) mu = chc.kn[t] > 0.f ? be / chc.kn[t] : 0.f;
      else mu = -kInf;
      sm.key[rank_slot<C>(t)] = t < sinks ? ~0u : ((ordered(mu) & ~0xFFu) | (uint32_t)t);
    };

    // ---- 2. surprise against the rows before the chunk: each workgroup's
    // best over its own rows, then (P > 1) the exchange of those bests
    if (tid == 0) sm.xok = 1;
    if constexpr (!PART) {
      cos_best<T, C, PART>(sm, chc, unit, &ul[0][0], LB, ntl, eb, ee, p, psh, pre, [] {}, [&](int t, float v, int r) {
        sm.bE[t] = v;
        sm.rE[t] = r;
      });
      lds_barrier();
    } else {
      // Exchange of the P workgroups' bests.  Each token's best is published
      // as one 64-bit record: key bits | (row (24 bits, all ones for none) |
      // step tag << 24) << 32, in the buffer of this step's parity; the tag
      // is 0x80 | (j mod 128), never 0, the value the buffer is cleared to at
      // state creation and reset.  Readers poll the records themselves until
      // all carry this step's tag, so the exchange is one store and one load
      // round trip; a record is written and read whole (relaxed agent-scope
      // atomics, coherent across the chip), and the tag tells it from the one
      // of two steps back.  (A
      // workgroup overwrites a slot two steps later only after it has read
      // every other workgroup's records of the step between, which they
      // publish after reading this one.)  The combine order does not matter:
      // (larger key, then lower row) is a total order.
      // The thread that combines a token's best over this workgroup's waves
      // publishes its record at once.
      uint64_t* xb = reinterpret_cast<uint64_t*>(d.xbuf) + ((size_t)s * 2 + (j & 1)) * ((size_t)m.P * C);
      const uint32_t tag = 0x80u | (uint32_t)(j & 0x7F);
      // Every thread settles the next chunk's loads after its tile loop, ahead
      // of the record stores: loads and stores retire in order, so a wait for
      // those registers after the stores (in the chunk store below) would also
      // wait for the stores to reach the device-coherent level.
      // The first four waves also write the previous step's index list there:
      // each SIMD's older wave issues first and ends its tile loop well before
      // the other, so these writes fill the gap before the combine's barrier.
      auto settle = [&] {
        if constexpr (kEarly) {
#pragma unroll
          for (int i = 0; i < ChunkRegs<T, C>::NK; ++i) asm volatile("" : "+v"(cr.k[i]));
#pragma unroll
          for (int i = 0; i < ChunkRegs<T, C>::NV; ++i) asm volatile("" : "+v"(cr.v[i]));
          asm volatile("" : "+v"(cr.l));
        }
        constexpr int kFirst = kScanThreads / 2;   // the first four waves
        if (j > j_begin && tid < kFirst)
          for_own_rows(R0, [&](int q, int r) { idx[prev_off + r] = sm.ver_cur[q]; }, kFirst);
      };
      cos_best<T, C, PART>(sm, chc, unit, &ul[0][0], LB, ntl, eb, ee, p, psh, pre, settle, [&](int t, float v, int r) {
        const uint32_t rr24 = r == INT_MAX ? 0xFFFFFFu : (uint32_t)r;
        const uint64_t x = (uint64_t)__float_as_uint(v) | ((uint64_t)(rr24 | (tag << 24)) << 32);
        __hip_atomic_store(xb + (size_t)p * C + t, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      });
      // XL lanes per token (a power of two, at most 8): lane sub polls the
      // records of workgroups sub, sub + XL, ...; the group then combines.
      // The first poll is issued before the next chunk's LDS store, which
      // runs while it travels.
      constexpr int XL = kScanThreads / C < 8 ? kScanThreads / C : 8;
      constexpr int XR = (8 + XL - 1) / XL;   // records per lane at most
      const int xt = tid / XL, xs = tid % XL;
      uint32_t pending = 0u;
      if (xt < C) {
#pragma unroll
        for (int i = 0; i < XR; ++i) {
          const int q = xs + XL * i;
          if (q < m.P) pending |= 1u << i;
        }
      }
      uint64_t x[XR];
      auto poll = [&] {
#pragma unroll
        for (int i = 0; i < XR; ++i)
          if (pending & (1u << i))
            x[i] = __hip_atomic_load(xb + (size_t)(xs + XL * i) * C + xt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      };
      poll();
      if constexpr (kEarly)
        if (j + 1 < j_end) chunk_store<T, C>(cr, sm.ch[cur ^ 1], m.no_gate);
      float v = 0.f;
      int r = INT_MAX;
      for (int spin = 0; pending != 0u;) {
#pragma unroll
        for (int i = 0; i < XR; ++i) {
          if ((pending & (1u << i)) && (uint32_t)(x[i] >> 56) == tag) {
            pending &= ~(1u << i);
            const float ov = __uint_as_float((uint32_t)x[i]);
            const uint32_t rr = (uint32_t)(x[i] >> 32) & 0xFFFFFFu;
            const int orow = rr == 0xFFFFFFu ? INT_MAX : (int)rr;
            if (ov > v || (ov == v && orow < r)) { v = ov; r = orow; }
          }
        }
        if (pending != 0u) {
          if (++spin >= kSpinLimit) {
            sm.xok = 0;
            __hip_atomic_store(d.xerr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
          }
          __builtin_amdgcn_s_sleep(1);
          poll();
        }
      }
      if (xt < C) {   // (every lane of a token's group is here)
        auto take = [&](float ov, int orow) {
          if (ov > v || (ov == v && orow < r)) { v = ov; r = orow; }
        };
        if constexpr (XL >= 2) take(__int_as_float(xor_lane<1>(__float_as_int(v))), xor_lane<1>(r));
        if constexpr (XL >= 4) take(__int_as_float(xor_lane<2>(__float_as_int(v))), xor_lane<2>(r));
        if constexpr (XL >= 8) take(__int_as_float(xor_lane<4>(__float_as_int(v))), xor_lane<4>(r));
        if (xs == 0) token_key(xt, v, r);
      }
      wait_vmem();   // this workgroup's global writes of the previous step, before the row loads below
      lds_barrier();
      if (!sm.xok) break;   // the whole workgroup leaves the chunk loop
    }
    // With the index lists in global memory, the new list starts as a copy of
    // the previous one; the update overwrites the rows it touches.  (Each wave
    // waits for its copies to complete, so the overwrites come after them.)
    if (!ver_lds && j > 0) {
      for (int i = tid; i < R0; i += kScanThreads)
        if (own(i)) idx[ioff + i] = idx[prev_off + i];
      wait_vmem();
    }
    // Otherwise the next chunk loads from here to the end of the step (issued
    // after the pass: loads complete in order, so a wait for the pass's tiles
    // would also wait for these).
    if constexpr (!kEarly)
      if (j + 1 < j_end) chunk_load<T, C>(cr, m, src, s, P0 + C, ring_k, ring_v, ring_l);
    // (the row-split kernel's exchange has already done this for every token)
    if constexpr (!PART) {
      for (int t = tid; t < C; t += kScanThreads) token_key(t, sm.bE[t], sm.rE[t]);
      lds_barrier();
    }

    // ---- 3. append the m_j most surprising candidates.  Up to C = 128 the
    // lane that reports a token's rank marks the token in the chunk's append
    // mask, whose bits in position order are the appended tokens in order.
    // Beyond, that lane also places the token: a wave's reporting lanes hold
    // consecutive tokens in lane order, so a ballot and the per-wave counts
    // give each appended token its place in position order.  Without appends
    // (a full fixed or saturated state) every non-sink token merges and no
    // rank is needed (m_j is the same for the whole workgroup).
    constexpr bool kAM = C <= 128;
    if (mj > 0) {
      int t;
      const int rank = parallel_rank<C>(sm.key, t);
      const bool ap = rank >= 0 && t >= sinks && rank < mj;
      if constexpr (kAM) {
        if (ap) __hip_atomic_fetch_or(&sm.amask[t >> 5], 1u << (t & 31), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      } else {
        const unsigned long long bal = __ballot(ap);
        const int within = __popcll(bal & ((1ull << lane) - 1ull));
        if (lane == 0) sm.wtot[w] = __popcll(bal);
        lds_barrier();
        int off = 0;
        for (int ww = 0; ww < w; ++ww) off += sm.wtot[ww];
        if (rank >= 0) {
          sm.flag[t] = t < sinks ? kSink : (ap ? kAppend : kMerge);
          if (ap) {
            sm.arow[t] = R0 + sinks + off + within;
            sm.app_list[off + within] = t;
          }
        }
      }
      lds_barrier();
    }

    // ---- 4. best against the new rows (their key sums are the creating tokens'
    // live keys, in LDS: dot(k_t, k_s) / |k_s|), then the winner-take-all assignment.
    // New row R0 + e was created by token e (a sink, e < sinks) or by the
    // (e - sinks)-th appended token; sink rows are candidates only unprotected.
    // The lane group of token t (four lanes) takes the token's kind and row
    // (every lane computes them; lane 0 publishes them) and keeps them for the
    // update; when a merged token's target is one of this workgroup's rows it
    // starts loading that row (sums, count, radius) into its registers: the
    // group updates the row below if t comes first on it (the row's values
    // from the previous steps).
    const int e0 = m.unprot ? 0 : sinks;
    const bool new_rows = nc > e0;   // candidates among this step's new rows (uniform)
    const int fallback = ee > eb ? eb : (R0 + sinks);
    constexpr int AW = C / 32;
    uint32_t am[kAM ? AW : 1];
    if constexpr (kAM) {
#pragma unroll
      for (int i = 0; i < AW; ++i) am[i] = __builtin_amdgcn_readfirstlane(sm.amask[i]);   // uniform
    }
    // (append mask) the creating token of new row e0 + lane, for the first 64
    int crl = 0;
    if constexpr (kAM) {
      const int el = e0 + lane;
      if (el < nc) crl = el < sinks ? el : kth_bit<AW>(am, el - sinks);
    }
    RowRegs rr[TP];
    int kind[TP], arow_r[TP];
#pragma unroll
    for (int ps = 0; ps < TP; ++ps) {
      const int t = (tid >> 2) + ps * (kScanThreads / 4);
      const int sub = tid & 3;
      kind[ps] = kSink;
      arow_r[ps] = 0;
      if (t >= C) continue;   // the same for the whole lane group
      bool ap;
      if constexpr (kAM) ap = t >= sinks && ((am[t >> 5] >> (t & 31)) & 1u);
      else ap = mj > 0 && t >= sinks && sm.flag[t] == kAppend;
      const bool merged = t >= sinks && !ap;
      // the token's best existing row, read before the new-row pass so that
      // the reads overlap it
      const int rEt = sm.rE[t];
      const float bEt = sm.bE[t];
      float best = -kInf;
      int brow = INT_MAX;
      if (new_rows && (kAM || merged)) {
        // (with the append mask every lane group runs this, so that the
        // shuffles below read active lanes; only a merged token's result is used)
        float kt[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) kt[i] = tof(Kc[t][i]);
        // lane sub takes the new rows e with e - e0 = sub mod 4, in order;
        // row e >= sinks was created by the (e - sinks)-th appended token
        for (int e = e0 + sub; e < nc; e += 4) {
          int s2 = e;
          if constexpr (kAM) {
            const int sh = __shfl(crl, (e - e0) & 63);
            if (e >= sinks) s2 = e - e0 < 64 ? sh : kth_bit<AW>(am, e - sinks);
          } else {
            if (e >= sinks) s2 = sm.app_list[e - sinks];
          }
          // four partial sums (dims i mod 4) keep the dependent chains short
          float dp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int i = 0; i < 32; ++i) dp[i & 3] = fmaf(kt[i], tof(Kc[s2][i]), dp[i & 3]);
          const float dot = (dp[0] + dp[1]) + (dp[2] + dp[3]);
          const float nk = chc.kn[s2];
          const float val = nk > 0.f ? dot * __builtin_amdgcn_rcpf(nk) : 0.f;   // 1 ulp
          if (val > best) { best = val; brow = R0 + e; }
        }
        float ob = xor_lane<1>(best);
        int orow = xor_lane<1>(brow);
        if (ob > best || (ob == best && orow < brow)) { best = ob; brow = orow; }
        ob = xor_lane<2>(best);
        orow = xor_lane<2>(brow);
        if (ob > best || (ob == best && orow < brow)) { best = ob; brow = orow; }
      }
      const int mslot = t + 4 * (t / (C / 4));
      int a;
      if (merged) {
        const bool eok = rEt != INT_MAX, aok = brow != INT_MAX;
        if (eok && (!aok || bEt >= best)) a = rEt;
        else if (aok) a = brow;
        else a = fallback;
        a = min(max(a, 0), rows_after - 1);
        if (sub == 0) {
          if constexpr (kTab) {
            if (own(a)) __hip_atomic_fetch_or(&sm.rmask[vslot(a)][t >> 5], 1u << (t & 31), __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_WORKGROUP);
          } else {
            sm.mrow[mslot] = a;
          }
        }
        if (own(a)) row_load(rr[ps], key_sum, val_sum, count, rho, a, sub);
      } else {
        if (t < sinks) {
          a = R0 + t;
        } else if constexpr (kAM) {   // appended: its place among the appended tokens
          int below = 0;
#pragma unroll
          for (int i = 0; i < AW; ++i) {
            const int lo = t - 32 * i;   // bits of word i below position t
            const uint32_t mk = lo >= 32 ? ~0u : (lo > 0 ? (1u << lo) - 1u : 0u);
            below += __popc(am[i] & mk);
          }
          a = R0 + sinks + below;
        } else {
          a = sm.arow[t];
        }
        if (!kTab && sub == 0) sm.mrow[mslot] = -1;
      }
      kind[ps] = t < sinks ? kSink : (ap ? kAppend : kMerge);
      arow_r[ps] = a;
      if (sub == 0) {
        sm.flag[t] = kind[ps];
        sm.arow[t] = a;
      }
    }
    lds_barrier();
    if (kAM && tid < AW) sm.amask[tid] = 0u;   // (read above, before the barrier; set again after the next ranking)

    // schedule entry of the next step: a scalar load, issued here so that it is
    // covered by this step's closing barrier rather than stalling an LDS barrier
    if (j + 1 < j_end) sc_next = sched[j + 1];

    // ---- 5. update every touched or created row.  The lane group of token t
    // (four lanes; lane sub owns key dims [8 sub, 8 sub + 8) and value dims
    // [16 sub, 16 sub + 16)) fills the row t creates, or updates the row t
    // merges into when t comes first on it in position order.  The row's
    // merged tokens are found by a scan of the chunk's targets (lane sub scans
    // positions [sub Q, sub Q + Q)) and added in position order; the row's new
    // read form becomes version nver + t.
    constexpr int Q = C / 4, QW = (Q + 31) / 32;
#pragma unroll
    for (int ps = 0; ps < TP; ++ps) {
      const int t = (tid >> 2) + ps * (kScanThreads / 4);
      const int sub = tid & 3;
      const int tc = min(t, C - 1);
      const bool merged = kind[ps] == kMerge;
      const int target = arow_r[ps];
      if (t >= C || !own(target)) continue;   // another workgroup's row (the same for the lane group)
      // the row's merged tokens, one bit per position (every lane of the group)
      uint32_t mw[kTab ? MW : 4 * QW];
      if constexpr (kTab) {
        // from the row's mask, which the assignment filled
        const int slot = vslot(target);
        if constexpr (MW == 4) {
          const u32x4 x = *reinterpret_cast<const u32x4*>(&sm.rmask[slot][0]);
#pragma unroll
          for (int i = 0; i < 4; ++i) mw[i] = x[i];
        } else {
#pragma unroll
          for (int i = 0; i < MW; ++i) mw[i] = sm.rmask[slot][i];
        }
        // a merged token heads its row when it is the row's lowest position
        if (merged) {
          if (target >= R0) continue;
          bool head = true;
#pragma unroll
          for (int i = 0; i < MW; ++i) {
            const uint32_t below = 32 * i + 32 <= t ? ~0u : (32 * i < t ? (1u << (t - 32 * i)) - 1u : 0u);
            head = head && (mw[i] & below) == 0u;
          }
          if (!head) continue;
        }
        clear_slot = slot;
      } else {
        // from a scan of the chunk's targets (lane sub scans positions [sub Q, sub Q + Q))
        uint32_t mk[QW];
#pragma unroll
        for (int q = 0; q < QW; ++q) mk[q] = 0u;
        {
          const u32x4* m4 = reinterpret_cast<const u32x4*>(sm.mrow + sub * (Q + 4));
#pragma unroll
          for (int i = 0; i < Q / 4; ++i) {
            const u32x4 x = m4[i];
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (x[e] == (uint32_t)target) mk[(4 * i + e) >> 5] |= 1u << ((4 * i + e) & 31);
          }
        }
        // a merged token heads its row unless a lower position merges into it too
        uint32_t low = 0u;
        {
          const int qt = tc / Q, bt = tc % Q;
#pragma unroll
          for (int q = 0; q < QW; ++q) {
            const int lo = bt - 32 * q;   // bits of this word below position t
            const uint32_t below = lo >= 32 ? ~0u : (lo > 0 ? (1u << lo) - 1u : 0u);
            low |= sub < qt ? mk[q] : (sub == qt ? (mk[q] & below) : 0u);
          }
          low |= (uint32_t)xor_lane<1>((int)low);
          low |= (uint32_t)xor_lane<2>((int)low);
        }
        // every lane of the group takes all four quarters' masks (quarter q,
        // word qw holds positions q Q + 32 qw + bit)
#pragma unroll
        for (int qw = 0; qw < QW; ++qw) {
          mw[0 * QW + qw] = (uint32_t)__builtin_amdgcn_mov_dpp((int)mk[qw], 0x00, 0xF, 0xF, false);
          mw[1 * QW + qw] = (uint32_t)__builtin_amdgcn_mov_dpp((int)mk[qw], 0x55, 0xF, 0xF, false);
          mw[2 * QW + qw] = (uint32_t)__builtin_amdgcn_mov_dpp((int)mk[qw], 0xAA, 0xF, 0xF, false);
          mw[3 * QW + qw] = (uint32_t)__builtin_amdgcn_mov_dpp((int)mk[qw], 0xFF, 0xF, 0xF, false);
        }
        if (merged && (low != 0u || target >= R0)) continue;   // the same for the whole group
      }
      const bool creates = !merged;
      const int row = target;
      alignas(16) float K[8];
      alignas(16) float V[16];
      int n;
      float rh;
      if (creates) {
        // new row: the creating token, unscaled; its value norm is the read radius
        float v2 = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) K[i] = tof(Kc[t][8 * sub + i]);
#pragma unroll
        for (int i = 0; i < 16; ++i) { V[i] = tof(Vc[t][16 * sub + i]); v2 = fmaf(V[i], V[i], v2); }
        v2 = quad_sum(v2);
        n = 1;
        rh = sqrtf(v2);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          K[i] = rr[ps].k[0][i];
          K[4 + i] = rr[ps].k[1][i];
#pragma unroll
          for (int q = 0; q < 4; ++q) V[4 * q + i] = rr[ps].v[q][i];
        }
        n = rr[ps].n;
        rh = rr[ps].rh;
      }
      // the merged tokens, added in position order, up to C = 128 two at a
      // time (both tokens' reads in flight together; a lone last token reads
      // itself twice)
      constexpr int NWD = kTab ? MW : 4 * QW;
#pragma unroll
      for (int wd = 0; wd < NWD; ++wd) {
        const int pbase = kTab ? 32 * wd : (wd / QW) * Q + 32 * (wd % QW);
        uint32_t mm = mw[wd];
        while (mm) {
          const int t1 = pbase + __builtin_ctz(mm);
          mm &= mm - 1u;
          const bool two = C <= 128 && mm != 0u;   // (registers: one at a time beyond)
          const int t2 = two ? pbase + __builtin_ctz(mm) : t1;
          if (two) mm &= mm - 1u;
          const float g1 = chc.g[t1], g2 = chc.g[t2];
          alignas(16) T k1[8], k2[8], v1[16], v2[16];
#pragma unroll
          for (int i = 0; i < 8; i += 16 / (int)sizeof(T)) {
            copy16(k1 + i, &Kc[t1][8 * sub + i]);
            copy16(k2 + i, &Kc[t2][8 * sub + i]);
          }
#pragma unroll
          for (int i = 0; i < 16; i += 16 / (int)sizeof(T)) {
            copy16(v1 + i, &Vc[t1][16 * sub + i]);
            copy16(v2 + i, &Vc[t2][16 * sub + i]);
          }
#pragma unroll
          for (int i = 0; i < 8; ++i) K[i] = fmaf(g1, tof(k1[i]), K[i]);
#pragma unroll
          for (int i = 0; i < 16; ++i) V[i] = fmaf(g1, tof(v1[i]), V[i]);
          if (two) {
#pragma unroll
            for (int i = 0; i < 8; ++i) K[i] = fmaf(g2, tof(k2[i]), K[i]);
#pragma unroll
            for (int i = 0; i < 16; ++i) V[i] = fmaf(g2, tof(v2[i]), V[i]);
          }
          n += two ? 2 : 1;
        }
      }
      {
        float* ks = key_sum + (size_t)row * 32 + 8 * sub;
        float* vs = val_sum + (size_t)row * 64 + 16 * sub;
#pragma unroll
        for (int i = 0; i < 8; i += 4) *reinterpret_cast<float4*>(ks + i) = *reinterpret_cast<const float4*>(&K[i]);
#pragma unroll
        for (int i = 0; i < 16; i += 4) *reinterpret_cast<float4*>(vs + i) = *reinterpret_cast<const float4*>(&V[i]);
      }
      if (sub == 0) {
        count[row] = n;
        rho[row] = rh;
      }
      // the row's unit key direction (both copies) and its read form, version nver + t
      const int ver = nver + t;
      bf16* ulrow = nullptr;
      if constexpr (Is<T>::bf && NL > 0) {
        if (row >= LB) {
          const int ls = own_slot(row, LB, psh);
          if (ls < NL) ulrow = &ul[ls][0];
        }
      }
      float rs, vsc;
      row_derive<T>(K, V, n, rh, sub, m, unit + (size_t)row * 128, ulrow, kread + (size_t)row * 32,
                    vread + (size_t)row * 64, pkey + (size_t)ver * 32, pval + (size_t)ver * 64, rs, vsc);
      if (sub == 0) {
        prho[ver] = rh;
        pcount[ver] = n;
        d.pnorm[(size_t)s * m.V_cap + ver] = make_float2(rs, vsc);
        if (ver_lds) sm.ver_cur[vslot(row)] = ver;
        else idx[ioff + row] = ver;
      }
    }
    if (m.trace && p == 0) {
      int* tslot = d.tslot + (size_t)s * m.max_tokens;
      uint8_t* tkind = d.tkind + (size_t)s * m.max_tokens;
      for (int t = tid; t < C; t += kScanThreads) {
        tslot[P0 + t] = sm.arow[t];
        tkind[P0 + t] = (uint8_t)sm.flag[t];
      }
    }
    // the next chunk into the spare buffer (chunk j - 1's, no longer read)
    if constexpr (NBUF == 2 && !kEarly)
      if (j + 1 < j_end) chunk_store<T, C>(cr, sm.ch[cur ^ 1], m.no_gate);
    nver += C;
    prev_off = (int)ioff;
    last_rows = rows_after;
    // Publish the next chunk's buffer and the step's writes.  The row-split
    // kernel reads none of this step's global writes before the next step's
    // exchange (its unit directions come from LDS), so it needs only an LDS
    // barrier here; each thread waits for its stores before the barrier that
    // closes the exchange, by when they have long completed.
    if constexpr (PART) lds_barrier();
    else __syncthreads();
  }
  if (ver_lds && j_end > j_begin) for_own_rows(last_rows, [&](int q, int r) { idx[prev_off + r] = sm.ver_cur[q]; });
  if (tid == 0 && p == 0) d.nver[s] = nver;
}

// =====================================================================
// Attention over [state read form || window], one workgroup per (sequence,
// query chunk), one wave per 32 queries.
// [KVM summary, Methodology]: a single softmax attention layer.
// [KVM summary, Core mechanisms 4]: state keys have a zero rotary subspace and
//   meet the unrotated query (only the 32 live dims contract); window keys are
//   rotated and meet the rotated query.
// S^T = K . Q^T is computed so that each lane owns one query: the softmax row
// statistics are lane-local plus one exchange with lane l^32, and P^T comes
// out of the D layout already in the B-operand layout of O^T = V^T . P^T.
// =====================================================================
template <typename T>
struct AttnCfg {
  static constexpr int KSTR = Is<T>::bf ? 72 : 68;  // sK row stride (elements)
  static constexpr int VSTR = Is<T>::bf ? 68 : 65;  // sVt row stride (elements)
};

// RoPE of a pair (x, y) = (dim j, dim j+16).
__device__ __forceinline__ void rot(float& x, float& y, float c, float s) {
  const float a = x * c - y * s;
  const float b = y * c + x * s;
  x = a;
  y = b;
}

// State tile: rows r0..r0+63 of the snapshot (version ids in idxl).  Stages the
// read-form key (live dims) into sK and the read-form value rho * u transposed
// into sVt.  Rows past S are zero.
template <typename T, int NT>
__device__ void stage_state(void* sKv, T* sVt, const int* idxl, const typename Rd<T>::type* pk, const T* pv, int r0,
                            int S) {
  using RT = typename Rd<T>::type;
  RT* sK = reinterpret_cast<RT*>(sKv);
  constexpr int KSTR = AttnCfg<T>::KSTR, VSTR = AttnCfg<T>::VSTR;
  constexpr int EL = 16 / sizeof(RT);
  constexpr int KPC = 32 / EL;  // pieces per live key row
  for (int task = threadIdx.x; task < 64 * KPC; task += NT) {
    const int i = task / KPC, p = task % KPC;
    const int r = r0 + i;
    RT* dst = sK + i * KSTR + p * EL;
    if (r < S) copy16(dst, pk + (size_t)idxl[r] * 32 + p * EL);
    else zero16(dst);
  }
  constexpr int VG = 64 / EL;  // dim groups
  for (int task = threadIdx.x; task < 32 * VG; task += NT) {
    const int rp = task / VG, dg = task % VG;
    const int i0 = 2 * rp;
    alignas(16) T a[EL];
    alignas(16) T b[EL];
    const int r = r0 + i0;
    if (r < S) copy16(a, pv + (size_t)idxl[r] * 64 + dg * EL);
    else zero16(a);
    if (r + 1 < S) copy16(b, pv + (size_t)idxl[r + 1] * 64 + dg * EL);
    else zero16(b);
#pragma unroll
    for (int e = 0; e < EL; ++e) {
      T* dst = sVt + (dg * EL + e) * VSTR + i0;
      dst[0] = a[e];
      dst[1] = b[e];
    }
  }
}

template <typename T, int NT>
__device__ void stage_window(T* sK, T* sVt, int64_t k0, int64_t hi, const Src& src, int s, const T* ring_k,
                             const T* ring_v, int R, const float* rc, const float* rsn) {
  constexpr int KSTR = AttnCfg<T>::KSTR, VSTR = AttnCfg<T>::VSTR;
  constexpr int EL = 16 / sizeof(T);
  constexpr int RT_ = 16 / EL;      // rotary tasks per key (each: EL dims + their partners)
  constexpr int PT = 32 / EL;       // plain pieces per key (dims 32..63)
  constexpr int KT = RT_ + PT;
  for (int task = threadIdx.x; task < 64 * KT; task += NT) {
    const int i = task / KT, p = task % KT;
    const int64_t pos = k0 + i;
    T* row = sK + i * KSTR;
    if (pos >= hi) {
      if (p < RT_) { zero16(row + p * EL); zero16(row + 16 + p * EL); }
      else zero16(row + 32 + (p - RT_) * EL);
      continue;
    }
    if (pos >= src.p0) {
      const T* kr = reinterpret_cast<const T*>(src.k) + ((size_t)s * src.n_call + (size_t)(pos - src.p0)) * 64;
      if (p < RT_) {
        alignas(16) T x[EL];
        alignas(16) T y[EL];
        copy16(x, kr + p * EL);
        copy16(y, kr + 16 + p * EL);
#pragma unroll
        for (int e = 0; e < EL; ++e) {
          float a = tof(x[e]), b = tof(y[e]);
          rot(a, b, rc[pos * 16 + p * EL + e], rsn[pos * 16 + p * EL + e]);
          x[e] = fromf<T>(a);
          y[e] = fromf<T>(b);
        }
        copy16(row + p * EL, x);
        copy16(row + 16 + p * EL, y);
      } else {
        copy16(row + 32 + (p - RT_) * EL, kr + 32 + (p - RT_) * EL);
      }
    } else {
      const T* kr = ring_k + (size_t)(pos % R) * 64;  // ring keys are already rotated
      if (p < RT_) { copy16(row + p * EL, kr + p * EL); copy16(row + 16 + p * EL, kr + 16 + p * EL); }
      else copy16(row + 32 + (p - RT_) * EL, kr + 32 + (p - RT_) * EL);
    }
  }
  constexpr int VG = 64 / EL;
  for (int task = threadIdx.x; task < 32 * VG; task += NT) {
    const int rp = task / VG, dg = task % VG;
    const int i0 = 2 * rp;
    alignas(16) T a[EL];
    alignas(16) T b[EL];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int64_t pos = k0 + i0 + q;
      T* dstv = q ? b : a;
      if (pos >= hi) { zero16(dstv); continue; }
      const T* vr = pos >= src.p0
                        ? reinterpret_cast<const T*>(src.v) + ((size_t)s * src.n_call + (size_t)(pos - src.p0)) * 64
                        : ring_v + (size_t)(pos % R) * 64;
      copy16(dstv, vr + dg * EL);
    }
#pragma unroll
    for (int e = 0; e < EL; ++e) {
      T* dst = sVt + (dg * EL + e) * VSTR + i0;
      dst[0] = a[e];
      dst[1] = b[e];
    }
  }
}

// 8 values of a transposed tile row: keys {kb+4h..kb+4h+3, kb+8+4h..kb+8+4h+3} (+16 for the second step).
template <typename V8, typename V4, typename E>
__device__ __forceinline__ V8 vfrag(const E* vr, int off) {
  const V4 a = *reinterpret_cast<const V4*>(vr + off);
  const V4 b = *reinterpret_cast<const V4*>(vr + off + 8);
  return V8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

template <typename T, int NW>
__global__ __launch_bounds__(NW * 64) void attn_kernel(Dims m, Dev d, Src src, int64_t c_begin, int n_q,
                                                       int64_t end_pos, T* out) {
  using RT = typename Rd<T>::type;
  constexpr bool BF = Is<T>::bf;
  constexpr int C = NW * 32;
  constexpr int NT = NW * 64;
  constexpr int KSTR = AttnCfg<T>::KSTR, VSTR = AttnCfg<T>::VSTR;
  static_assert(sizeof(RT) == sizeof(T), "read-form and input types share the LDS tile layout");
  __shared__ __attribute__((aligned(16))) T sK[64 * KSTR];
  __shared__ __attribute__((aligned(16))) T sVt[64 * VSTR];

  // Block -> (sequence, chunk).  Consecutive block ids land on consecutive XCDs;
  // keep every chunk of a sequence on one XCD (its state rows stay in that L2)
  // and hand out the longest chunks (largest state, full window) first.
  int s, cl;
  {
    const int b = blockIdx.x;
    if (m.BH % 8 == 0) {
      const int x = b & 7, k = b >> 3, spx = m.BH >> 3;
      s = x + 8 * (k % spx);
      cl = n_q - 1 - k / spx;
    } else {
      s = b % m.BH;
      cl = n_q - 1 - b / m.BH;
    }
  }
  if (src.seq) {   // this sequence's own query chunks, input position and end
    const int64_t* sr = src.seq + (size_t)s * kSeqFields;
    if (cl >= (int)sr[kSeqNq]) return;
    src.p0 = sr[kSeqP0];
    c_begin = sr[kSeqCb];
    end_pos = sr[kSeqEnd];
  }
  const int64_t c = c_begin + cl;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, jl = lane & 31, h = lane >> 5;
  const int64_t cpos = c * C;
  const int64_t qpos = cpos + 32 * w + jl;
  const bool qvalid = qpos < end_pos;
  const int64_t qp = qvalid ? qpos : (end_pos - 1);
  const float sl2 = m.scale * kLog2e;

  // ---- query fragments (B operand of S^T = K . Q^T)
  const T* qrow = reinterpret_cast<const T*>(src.q) + ((size_t)s * src.n_call + (size_t)(qp - src.p0)) * 64;
  const float* rc = d.rope_cos + qp * 16;
  const float* rsn = d.rope_sin + qp * 16;
  bf16x8 qf[4];     // bf16 window: k-step kk holds dims 16kk + 8h + e (rotated for kk < 2)
  f16x8 qs16[2];    // bf16 path, state: dims 32 + 16kk + 8h + e in fp16 (scaled by 2^-qsh)
  float qw[32];     // fp32 window: dims 32h + kk
  float qs[16];     // fp32 state: dims 32 + 16h + kk
  float sl2_state = sl2;
  if constexpr (BF) {
    alignas(16) T x[4][8];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) copy16(x[kk], qrow + 16 * kk + 8 * h);
    float qmx = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float a = tof(x[0][e]), b = tof(x[1][e]);
      rot(a, b, rc[8 * h + e], rsn[8 * h + e]);
      qf[0][e] = (bf16)a;
      qf[1][e] = (bf16)b;
      qf[2][e] = x[2][e];
      qf[3][e] = x[3][e];
      qmx = fmaxf(qmx, fmaxf(fabsf(tof(x[2][e])), fabsf(tof(x[3][e]))));
    }
    // fp16 range guard: scale the query's live dims by an exact power of two
    // when they could overflow fp16; the state logits are scaled back.
    qmx = fmaxf(qmx, partner_f(qmx));
    int qsh = 0;
    if (qmx >= 16384.f) {
      int ex;
      frexpf(qmx, &ex);
      qsh = ex - 14;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      qs16[0][e] = (f16)ldexpf(tof(x[2][e]), -qsh);
      qs16[1][e] = (f16)ldexpf(tof(x[3][e]), -qsh);
    }
    sl2_state = ldexpf(sl2, qsh);
  } else {
#pragma unroll
    for (int kk = 0; kk < 32; ++kk) qw[kk] = tof(qrow[32 * h + kk]);
    if (h == 0) {
#pragma unroll
      for (int e = 0; e < 16; ++e) rot(qw[e], qw[16 + e], rc[e], rsn[e]);
    }
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) qs[kk] = tof(qrow[32 + 16 * h + kk]);
  }

  float mrun = -kInf, lrun = 0.f;
  f32x16 O0 = {}, O1 = {};

  // Online softmax over one 32-key subtile: scales acc into log2 units, masks
  // invalid keys, updates the running max / sum, rescales O, returns p.
  auto softmax_step = [&](const f32x16& acc, float scl, auto valid, float (&p)[16]) {
    float sc[16];
    float mx = -kInf;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      sc[r] = valid(8 * (r >> 2) + 4 * h + (r & 3)) ? acc[r] * scl : -kInf;
      mx = fmaxf(mx, sc[r]);
    }
    mx = fmaxf(mx, partner_f(mx));
    const float mnew = fmaxf(mrun, mx);
    const float muse = mnew == -kInf ? 0.f : mnew;
    const float alpha = exp2_fast(mrun - muse);
    float ps = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) { p[r] = exp2_fast(sc[r] - muse); ps += p[r]; }
    lrun = lrun * alpha + ps;
    mrun = mnew;
#pragma unroll
    for (int r = 0; r < 16; ++r) { O0[r] *= alpha; O1[r] *= alpha; }
  };

  // ---- state part: the state after absorbing chunk c - W/C - 1
  const int64_t jj = c - m.W / C - 1;
  int S = 0;
  int64_t ioff = 0;
  if (jj >= 0) {
    const int4 sc4 = d.sched[jj];
    S = sc4.z + sc4.x + sc4.y;
    ioff = sc4.w;
  }
  const int* idxl = d.idx + (size_t)s * m.idx_total + ioff;
  const RT* pk = reinterpret_cast<const RT*>(d.pkey) + (size_t)s * m.V_cap * 32;
  const T* pv = reinterpret_cast<const T*>(d.pval) + (size_t)s * m.V_cap * 64;
  for (int r0 = 0; r0 < S; r0 += 64) {
    __syncthreads();
    stage_state<T, NT>(sK, sVt, idxl, pk, pv, r0, S);
    __syncthreads();
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int kb = 32 * sub;
      if (r0 + kb >= S) continue;
      const int lim = S - r0 - kb;  // valid rows in this subtile
      const RT* kr = reinterpret_cast<const RT*>(sK) + (kb + jl) * KSTR;
      f32x16 acc = {};
      if constexpr (BF) {
        acc = mfma_f16(*reinterpret_cast<const f16x8*>(kr + 8 * h), qs16[0], acc);
        acc = mfma_f16(*reinterpret_cast<const f16x8*>(kr + 16 + 8 * h), qs16[1], acc);
      } else {
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) acc = mfma_f32(kr[16 * h + kk], qs[kk], acc);
      }
      float p[16];
      softmax_step(acc, sl2_state, [&](int key) { return key < lim; }, p);
      if constexpr (BF) {
        bf16x8 pf0, pf1;
#pragma unroll
        for (int e = 0; e < 8; ++e) { pf0[e] = (bf16)p[e]; pf1[e] = (bf16)p[8 + e]; }
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) {
          const T* vr = sVt + (32 * dt + jl) * VSTR + kb;
          f32x16& O = dt ? O1 : O0;
          O = mfma_bf16(vfrag<bf16x8, bf16x4>(vr, 4 * h), pf0, O);
          O = mfma_bf16(vfrag<bf16x8, bf16x4>(vr, 16 + 4 * h), pf1, O);
        }
      } else {
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) {
          const T* vr = sVt + (32 * dt + jl) * VSTR + kb;
          f32x16& O = dt ? O1 : O0;
#pragma unroll
          for (int r = 0; r < 16; ++r) O = mfma_f32(vr[8 * (r >> 2) + 4 * h + (r & 3)], p[r], O);
        }
      }
    }
  }

  // ---- window part: keys [max(0, cC - W), min(cC + C, end)), causal
  const int64_t lo = cpos - m.W > 0 ? cpos - m.W : 0;
  const int64_t hi = cpos + C < end_pos ? cpos + C : end_pos;
  const int64_t qlast = min(cpos + 32 * w + 31, end_pos - 1);
  const T* ring_k = reinterpret_cast<const T*>(d.ring_k) + (size_t)s * m.R * 64;
  const T* ring_v = reinterpret_cast<const T*>(d.ring_v) + (size_t)s * m.R * 64;
  for (int64_t k0 = lo; k0 < hi; k0 += 64) {
    __syncthreads();
    stage_window<T, NT>(sK, sVt, k0, hi, src, s, ring_k, ring_v, m.R, d.rope_cos, d.rope_sin);
    __syncthreads();
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int kb = 32 * sub;
      const int64_t ks = k0 + kb;
      if (ks >= hi || ks > qlast) continue;
      const T* kr = sK + (kb + jl) * KSTR;
      f32x16 acc = {};
      if constexpr (BF) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          acc = mfma_bf16(*reinterpret_cast<const bf16x8*>(kr + 16 * kk + 8 * h), qf[kk], acc);
      } else {
#pragma unroll
        for (int kk = 0; kk < 32; ++kk) acc = mfma_f32(kr[32 * h + kk], qw[kk], acc);
      }
      float p[16];
      softmax_step(acc, sl2, [&](int key) { const int64_t kp = ks + key; return kp < hi && kp <= qpos; }, p);
      if constexpr (BF) {
        bf16x8 pf0, pf1;
#pragma unroll
        for (int e = 0; e < 8; ++e) { pf0[e] = (bf16)p[e]; pf1[e] = (bf16)p[8 + e]; }
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) {
          const T* vr = sVt + (32 * dt + jl) * VSTR + kb;
          f32x16& O = dt ? O1 : O0;
          O = mfma_bf16(vfrag<bf16x8, bf16x4>(vr, 4 * h), pf0, O);
          O = mfma_bf16(vfrag<bf16x8, bf16x4>(vr, 16 + 4 * h), pf1, O);
        }
      } else {
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) {
          const T* vr = sVt + (32 * dt + jl) * VSTR + kb;
          f32x16& O = dt ? O1 : O0;
#pragma unroll
          for (int r = 0; r < 16; ++r) O = mfma_f32(vr[8 * (r >> 2) + 4 * h + (r & 3)], p[r], O);
        }
      }
    }
  }

  // ---- normalise and store: lane holds dims 8*(r/4) + 4h + r%4 of its query
  const float lt = lrun + partner_f(lrun);
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;
  if (qvalid) {
    T* orow = out + ((size_t)s * src.n_call + (size_t)(qpos - src.p0)) * 64;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) {
      const f32x16& O = dt ? O1 : O0;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        alignas(16) T vals[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) vals[e] = fromf<T>(O[4 * g4 + e] * inv);
        T* dst = orow + 32 * dt + 8 * g4 + 4 * h;
        if constexpr (BF) {
          *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<const uint2*>(vals);
        } else {
          *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(vals);
        }
      }
    }
  }
}

// =====================================================================
// Pipelined bf16 attention (chunks of 128 or 256 queries).
// Same contraction layout as attn_kernel; what changes is the schedule:
//   * the snapshot's version list is preloaded into LDS;
//   * 64-key tiles are double-buffered: the global loads of tile T+1 are
//     issued into registers before tile T is computed and written to the
//     other LDS buffer after it, with one LDS-only barrier per tile;
//   * softmax in log2 units with scale*log2(e) folded into the query, the
//     running max fed to the MFMA as its C operand (the accumulator comes out
//     as logit - max), and a lazy rescale: the reference max moves only when
//     a tile exceeds it by more than 2^kTau;
//   * rho_i / rho_max is folded into the staged state values.
// =====================================================================
constexpr int kIdxCap = 4096;   // snapshot version ids kept in LDS
constexpr float kTau = 8.0f;    // lazy-rescale threshold (log2 units): p <= 2^8 in bf16/fp16

template <int NW>
__global__ __launch_bounds__(NW * 64, 2) void attn_bf16_kernel(Dims m, Dev d, Src src, int64_t c_begin, int n_q,
                                                            int64_t end_pos, bf16* out) {
  constexpr int C = NW * 32;
  constexpr int NT = NW * 64;
  constexpr int KSTR = 72, VSTR = 68;   // padded LDS strides (2-byte elements)
  static_assert(NT >= 256, "one staging task per thread");
  __shared__ __attribute__((aligned(16))) uint16_t sK[2][64 * KSTR];
  __shared__ __attribute__((aligned(16))) uint16_t sVt[2][64 * VSTR];
  __shared__ int sIdx[kIdxCap];

  int s, cl;
  {
    const int b = blockIdx.x;
    if (m.BH % 8 == 0) {
      const int x = b & 7, k = b >> 3, spx = m.BH >> 3;
      s = x + 8 * (k % spx);
      cl = n_q - 1 - k / spx;
    } else {
      s = b % m.BH;
      cl = n_q - 1 - b / m.BH;
    }
  }
  if (src.seq) {   // this sequence's own query chunks, input position and end
    const int64_t* sr = src.seq + (size_t)s * kSeqFields;
    if (cl >= (int)sr[kSeqNq]) return;
    src.p0 = sr[kSeqP0];
    c_begin = sr[kSeqCb];
    end_pos = sr[kSeqEnd];
  }
  const int64_t c = c_begin + cl;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, jl = lane & 31, h = lane >> 5;
  const int64_t cpos = c * C;
  const int64_t qpos = cpos + 32 * w + jl;
  const bool qvalid = qpos < end_pos;
  const int64_t qp = qvalid ? qpos : (end_pos - 1);
  const float c2 = m.scale * kLog2e;

  // ---- snapshot of chunk c - W/C - 1
  const int64_t jj = c - m.W / C - 1;
  int S = 0;
  int64_t ioff = 0;
  if (jj >= 0) {
    const int4 sc4 = d.sched[jj];
    S = sc4.z + sc4.x + sc4.y;
    ioff = sc4.w;
  }
  const int* idxg = d.idx + (size_t)s * m.idx_total + ioff;
  const bool idx_lds = S <= kIdxCap;
  if (idx_lds)
    for (int i = tid; i < S; i += NT) sIdx[i] = idxg[i];
  const f16* pk = reinterpret_cast<const f16*>(d.pkey) + (size_t)s * m.V_cap * 32;
  const bf16* pv = reinterpret_cast<const bf16*>(d.pval) + (size_t)s * m.V_cap * 64;

  // ---- query fragments (B operand of S^T = K . Q^T), pre-scaled by scale*log2(e)
  const bf16* qrow = reinterpret_cast<const bf16*>(src.q) + ((size_t)s * src.n_call + (size_t)(qp - src.p0)) * 64;
  bf16x8 qf[4];    // window: k-step kk holds dims 16kk + 8h + e (rotated for kk < 2)
  f16x8 qs16[2];   // state: dims 32 + 16kk + 8h + e, fp16, scaled by 2^-qsh
  int qsh = 0;
  {
    alignas(16) bf16 x[4][8];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) copy16(x[kk], qrow + 16 * kk + 8 * h);
    const float* rc = d.rope_cos + qp * 16;
    const float* rsn = d.rope_sin + qp * 16;
    float qmx = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float a = tof(x[0][e]), b = tof(x[1][e]);
      rot(a, b, rc[8 * h + e], rsn[8 * h + e]);
      qf[0][e] = (bf16)(a * c2);
      qf[1][e] = (bf16)(b * c2);
      qf[2][e] = (bf16)(tof(x[2][e]) * c2);
      qf[3][e] = (bf16)(tof(x[3][e]) * c2);
      qmx = fmaxf(qmx, fmaxf(fabsf(tof(x[2][e])), fabsf(tof(x[3][e]))) * c2);
    }
    // fp16 range guard for the state query: exact power-of-two pre-scale
    qmx = fmaxf(qmx, partner_f(qmx));
    if (qmx >= 16384.f) {
      int ex;
      frexpf(qmx, &ex);
      qsh = ex - 14;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      qs16[0][e] = (f16)ldexpf(tof(x[2][e]) * c2, -qsh);
      qs16[1][e] = (f16)ldexpf(tof(x[3][e]) * c2, -qsh);
    }
  }
  const bool wave_qsh = __ballot(qsh != 0) != 0ull;

  // ---- running softmax state: acc comes out of the MFMA as logit*c - mref
  float mref = 0.f, lrun = 0.f;
  bool started = false;
  f32x16 negm = {};
  f32x16 O0 = {}, O1 = {};

  // tile geometry: state tiles first, then window tiles
  const int n_st = (S + 63) >> 6;
  const int64_t lo = cpos - m.W > 0 ? cpos - m.W : 0;
  const int64_t hi = cpos + C < end_pos ? cpos + C : end_pos;
  const int n_wt = (int)((hi - lo + 63) >> 6);
  const int n_tiles = n_st + n_wt;
  const int64_t qlast = min(cpos + 32 * w + 31, end_pos - 1);
  const int64_t qfirst = cpos + 32 * w;
  const bf16* ring_k = reinterpret_cast<const bf16*>(d.ring_k) + (size_t)s * m.R * 64;
  const bf16* ring_v = reinterpret_cast<const bf16*>(d.ring_v) + (size_t)s * m.R * 64;

  // ---- staging: one K task and one V task per thread (threads >= 256 idle)
  const bool stager = tid < 256;
  const int ki = tid >> 2, kp = tid & 3;     // K task: key/row ki, part kp
  const int vrp = tid >> 3, vdg = tid & 7;   // V task: rows 2vrp, 2vrp+1; dims 8vdg..8vdg+7
  uint4 kr0, kr1, vr0, vr1;
  bool va_ok = false, vb_ok = false;
  int64_t k_pos = 0;   // window key position to rotate at commit (-1: no rotation)
  bool k_zero = false;

  auto row_version = [&](int r) -> int { return idx_lds ? sIdx[r] : idxg[r]; };
  auto issue = [&](int T) {
    if (!stager) return;
    if (T < n_st) {
      const int r0 = T << 6;
      const int r = r0 + ki;
      k_zero = r >= S;
      k_pos = -1;
      if (!k_zero) kr0 = *reinterpret_cast<const uint4*>(pk + (size_t)row_version(r) * 32 + 8 * kp);
      const int ra = r0 + 2 * vrp;
      va_ok = ra < S;
      vb_ok = ra + 1 < S;
      if (va_ok) vr0 = *reinterpret_cast<const uint4*>(pv + (size_t)row_version(ra) * 64 + 8 * vdg);
      if (vb_ok) vr1 = *reinterpret_cast<const uint4*>(pv + (size_t)row_version(ra + 1) * 64 + 8 * vdg);
    } else {
      const int64_t k0 = lo + ((int64_t)(T - n_st) << 6);
      const int64_t pos = k0 + ki;
      k_zero = pos >= hi;
      k_pos = -1;
      if (!k_zero) {
        const bool in = pos >= src.p0;
        const bf16* row = in ? reinterpret_cast<const bf16*>(src.k) + ((size_t)s * src.n_call + (size_t)(pos - src.p0)) * 64
                             : ring_k + (size_t)(pos % m.R) * 64;
        if (kp < 2) {
          kr0 = *reinterpret_cast<const uint4*>(row + 8 * kp);
          kr1 = *reinterpret_cast<const uint4*>(row + 16 + 8 * kp);
          if (in) k_pos = pos;   // ring keys are stored rotated
        } else {
          kr0 = *reinterpret_cast<const uint4*>(row + 32 + 16 * (kp - 2));
          kr1 = *reinterpret_cast<const uint4*>(row + 40 + 16 * (kp - 2));
        }
      }
      const int64_t pa = k0 + 2 * vrp;
      va_ok = pa < hi;
      vb_ok = pa + 1 < hi;
      if (pa < hi) {
        const bf16* row = pa >= src.p0 ? reinterpret_cast<const bf16*>(src.v) + ((size_t)s * src.n_call + (size_t)(pa - src.p0)) * 64
                                       : ring_v + (size_t)(pa % m.R) * 64;
        vr0 = *reinterpret_cast<const uint4*>(row + 8 * vdg);
      }
      if (pa + 1 < hi) {
        const bf16* row = pa + 1 >= src.p0 ? reinterpret_cast<const bf16*>(src.v) + ((size_t)s * src.n_call + (size_t)(pa + 1 - src.p0)) * 64
                                           : ring_v + (size_t)((pa + 1) % m.R) * 64;
        vr1 = *reinterpret_cast<const uint4*>(row + 8 * vdg);
      }
    }
  };
  auto commit = [&](int T, int buf) {
    if (!stager) return;
    uint16_t* K = sK[buf] + ki * KSTR;
    uint16_t* Vt = sVt[buf];
    if (T < n_st) {
      *reinterpret_cast<uint4*>(K + 8 * kp) = k_zero ? make_uint4(0, 0, 0, 0) : kr0;
    } else {
      uint4 x = kr0, y = kr1;
      if (k_zero) {
        x = make_uint4(0, 0, 0, 0);
        y = x;
      } else if (k_pos >= 0) {
        bf16* xa = reinterpret_cast<bf16*>(&x);
        bf16* ya = reinterpret_cast<bf16*>(&y);
        const float* rc = d.rope_cos + k_pos * 16 + 8 * kp;
        const float* rs = d.rope_sin + k_pos * 16 + 8 * kp;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float a = (float)xa[e], b = (float)ya[e];
          rot(a, b, rc[e], rs[e]);
          xa[e] = (bf16)a;
          ya[e] = (bf16)b;
        }
      }
      if (kp < 2) {
        *reinterpret_cast<uint4*>(K + 8 * kp) = x;
        *reinterpret_cast<uint4*>(K + 16 + 8 * kp) = y;
      } else {
        *reinterpret_cast<uint4*>(K + 32 + 16 * (kp - 2)) = x;
        *reinterpret_cast<uint4*>(K + 40 + 16 * (kp - 2)) = y;
      }
    }
    // values (state rho * u or window v, bf16), transposed (dim-major)
    const uint16_t* a = reinterpret_cast<const uint16_t*>(&vr0);
    const uint16_t* b = reinterpret_cast<const uint16_t*>(&vr1);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t pr = (va_ok ? (uint32_t)a[e] : 0u) | ((vb_ok ? (uint32_t)b[e] : 0u) << 16);
      *reinterpret_cast<uint32_t*>(Vt + (8 * vdg + e) * VSTR + 2 * vrp) = pr;
    }
  };

  // ---- online softmax over one 32-key subtile (acc = logit*c - mref; invalid keys already -inf)
  auto softmax_p = [&](f32x16& acc, float (&p)[16]) {
    float mx = acc[0];
#pragma unroll
    for (int r = 1; r < 15; r += 2) mx = fmaxf(fmaxf(mx, acc[r]), acc[r + 1]);
    mx = fmaxf(mx, acc[15]);
    mx = fmaxf(mx, partner_f(mx));
    if ((!started && mx != -kInf) || mx > kTau) {
      if (started) {
        const float alpha = exp2_fast(-mx);
        lrun *= alpha;
#pragma unroll
        for (int r = 0; r < 16; ++r) { O0[r] *= alpha; O1[r] *= alpha; }
      }
      mref += mx;
#pragma unroll
      for (int r = 0; r < 16; ++r) { acc[r] -= mx; negm[r] = -mref; }
      started = true;
    }
    float ps = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) { p[r] = exp2_fast(acc[r]); ps += p[r]; }
    lrun += ps;
  };

  auto compute = [&](int T, int buf) {
    const uint16_t* K = sK[buf];
    const uint16_t* Vt = sVt[buf];
    if (T < n_st) {
      const int r0 = T << 6;
#pragma unroll 1
      for (int sub = 0; sub < 2; ++sub) {
        const int kb = 32 * sub;
        if (r0 + kb >= S) continue;
        const int lim = S - r0 - kb;
        const f16* kr = reinterpret_cast<const f16*>(K) + (kb + jl) * KSTR;
        f32x16 acc;
        if (!wave_qsh) {
          acc = mfma_f16(*reinterpret_cast<const f16x8*>(kr + 8 * h), qs16[0], negm);
          acc = mfma_f16(*reinterpret_cast<const f16x8*>(kr + 16 + 8 * h), qs16[1], acc);
        } else {
          acc = mfma_f16(*reinterpret_cast<const f16x8*>(kr + 8 * h), qs16[0], f32x16{});
          acc = mfma_f16(*reinterpret_cast<const f16x8*>(kr + 16 + 8 * h), qs16[1], acc);
          const float sc = ldexpf(1.f, qsh);
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[r] = acc[r] * sc - mref;
        }
        if (lim < 32) {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (8 * (r >> 2) + 4 * h + (r & 3) >= lim) acc[r] = -kInf;
        }
        float p[16];
        softmax_p(acc, p);
        bf16x8 pf0, pf1;
#pragma unroll
        for (int e = 0; e < 8; ++e) { pf0[e] = (bf16)p[e]; pf1[e] = (bf16)p[8 + e]; }
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) {
          const bf16* vr = reinterpret_cast<const bf16*>(Vt) + (32 * dt + jl) * VSTR + kb;
          f32x16& O = dt ? O1 : O0;
          O = mfma_bf16(vfrag<bf16x8, bf16x4>(vr, 4 * h), pf0, O);
          O = mfma_bf16(vfrag<bf16x8, bf16x4>(vr, 16 + 4 * h), pf1, O);
        }
      }
    } else {
      const int64_t k0 = lo + ((int64_t)(T - n_st) << 6);
#pragma unroll 1
      for (int sub = 0; sub < 2; ++sub) {
        const int kb = 32 * sub;
        const int64_t ks = k0 + kb;
        if (ks >= hi || ks > qlast) continue;
        const bf16* kr = reinterpret_cast<const bf16*>(K) + (kb + jl) * KSTR;
        f32x16 acc = mfma_bf16(*reinterpret_cast<const bf16x8*>(kr + 8 * h), qf[0], negm);
#pragma unroll
        for (int kk = 1; kk < 4; ++kk)
          acc = mfma_bf16(*reinterpret_cast<const bf16x8*>(kr + 16 * kk + 8 * h), qf[kk], acc);
        if (ks + 31 >= hi || ks + 31 > qfirst) {
          // key ks + off is valid for this lane's query iff off < lim
          const int lim = (int)min(hi - ks, qpos - ks + 1);
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (8 * (r >> 2) + 4 * h + (r & 3) >= lim) acc[r] = -kInf;
        }
        float p[16];
        softmax_p(acc, p);
        bf16x8 pf0, pf1;
#pragma unroll
        for (int e = 0; e < 8; ++e) { pf0[e] = (bf16)p[e]; pf1[e] = (bf16)p[8 + e]; }
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) {
          const bf16* vr = reinterpret_cast<const bf16*>(Vt) + (32 * dt + jl) * VSTR + kb;
          f32x16& O = dt ? O1 : O0;
          O = mfma_bf16(vfrag<bf16x8, bf16x4>(vr, 4 * h), pf0, O);
          O = mfma_bf16(vfrag<bf16x8, bf16x4>(vr, 16 + 4 * h), pf1, O);
        }
      }
    }
  };

  // ---- pipeline: prologue stages tile 0; each iteration loads T+1, computes T, stages T+1
  __syncthreads();   // version ids in LDS
  if (n_tiles > 0) {
    issue(0);
    commit(0, 0);
  }
  lds_barrier();
  for (int T = 0; T < n_tiles; ++T) {
    if (T + 1 < n_tiles) issue(T + 1);
    compute(T, T & 1);
    if (T + 1 < n_tiles) commit(T + 1, (T + 1) & 1);
    lds_barrier();
  }

  // ---- normalise and store: lane holds dims 8*(r/4) + 4h + r%4 of its query
  const float lt = lrun + partner_f(lrun);
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;
  if (qvalid) {
    bf16* orow = out + ((size_t)s * src.n_call + (size_t)(qpos - src.p0)) * 64;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) {
      const f32x16& O = dt ? O1 : O0;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        alignas(8) bf16 vals[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) vals[e] = (bf16)(O[4 * g4 + e] * inv);
        *reinterpret_cast<uint2*>(orow + 32 * dt + 8 * g4 + 4 * h) = *reinterpret_cast<const uint2*>(vals);
      }
    }
  }
}

// =====================================================================
// Prefill attention, bf16, chunks of 128 / 256 (NW = C/32 waves of 32 queries).
// Every 64-key tile is staged by direct global->LDS transfers (no registers,
// no VALU): state rows are gathered from the row-version pool through the
// snapshot's index list (keys fp16, values rho * u bf16), window keys come
// pre-rotated (rotary dims from the RoPE prep buffer, live dims from k, or the
// ring for positions before this call).  LDS tiles are row-major with the
// 16-byte units of each row XOR-swizzled by the row index (applied through the
// source addresses), and the value operand of O^T = V^T . P^T is read with
// ds_read_b64_tr_b16, which returns 4 consecutive keys of one dim per lane.
// Two stages: the transfer of tile T+1 overlaps the MFMAs and softmax of T.
// [KVM summary, Core mechanisms 2, 4]; [KVM summary, Methodology].
// =====================================================================
constexpr int kDmaIdxCap = 8192;   // snapshot rows whose version ids fit the LDS list

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x4 ds_read_tr(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)(p));
}

// LDS swizzles of the staged attention tiles: a row's 16-byte unit u is
// stored at u XOR swz(row).  Each is chosen so that the lanes served in one
// LDS cycle hit distinct banks, whether a cycle serves 128 or 256 bytes:
//  - state keys (64-byte rows, ds_read_b128 by key row): the 8 or 16
//    consecutive rows of a cycle get distinct (row mod 2 or 4, unit) pairs;
//  - window keys (128-byte rows, ds_read_b128 by key row): likewise for
//    (row mod 1 or 2, unit) over 8 or 16 consecutive rows;
//  - values (128-byte rows, ds_read_b64_tr_b16): the 16 lanes of a cycle
//    read four rows two units each, so rows 0..3 (and 4..7) must land on
//    disjoint unit pairs.
// The previous row & mask swizzles measured ~50 M conflict cycles per
// 350M-workload launch; these measure none.
__device__ __forceinline__ int swz_sk(int r) { return ((r >> 2) & 1) | ((((r >> 1) ^ (r >> 3)) & 1) << 1); }
__device__ __forceinline__ int swz_wk(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int swz_v(int r) { return ((r & 3) << 1) | ((r >> 2) & 1); }

template <int NW>
__global__ __launch_bounds__(NW * 64, 3) void attn_dma_kernel(Dims m, Dev d, Src src, int64_t c_begin, int n_q,
                                                              int64_t end_pos, bf16* out) {
  constexpr int C = NW * 32;
  constexpr int NT = NW * 64;
  __shared__ __attribute__((aligned(16))) uint8_t sK0[8192];
  __shared__ __attribute__((aligned(16))) uint8_t sK1[8192];
  __shared__ __attribute__((aligned(16))) uint8_t sV0[8192];
  __shared__ __attribute__((aligned(16))) uint8_t sV1[8192];
  extern __shared__ int sIdx[];

  int s, cl;
  {
    const int b = blockIdx.x;
    if (m.BH % 8 == 0) {
      const int x = b & 7, k = b >> 3, spx = m.BH >> 3;
      s = x + 8 * (k % spx);
      cl = n_q - 1 - k / spx;
    } else {
      s = b % m.BH;
      cl = n_q - 1 - b / m.BH;
    }
  }
  if (src.seq) {   // this sequence's own query chunks, input position and end
    const int64_t* sr = src.seq + (size_t)s * kSeqFields;
    if (cl >= (int)sr[kSeqNq]) return;
    src.p0 = sr[kSeqP0];
    c_begin = sr[kSeqCb];
    end_pos = sr[kSeqEnd];
  }
  const int64_t c = c_begin + cl;
  const int tid = threadIdx.x, lane = tid & 63, jl = lane & 31, h = lane >> 5;
  // wave index, made uniform for the compiler: the LDS targets of the
  // global->LDS transfers (in M0) then come from scalar registers, with no
  // per-transfer loop over lanes
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t cpos = c * C;
  const int64_t qpos = cpos + 32 * w + jl;
  const bool qvalid = qpos < end_pos;
  const int64_t qp = qvalid ? qpos : (end_pos - 1);
  const float c2 = m.scale * kLog2e;

  // ---- snapshot of chunk c - W/C - 1: its version ids into LDS
  const int64_t jj = c - m.W / C - 1;
  int S = 0;
  int64_t ioff = 0;
  if (jj >= 0) {
    const int4 sc4 = d.sched[jj];
    S = sc4.z + sc4.x + sc4.y;
    ioff = sc4.w;
  }
  {
    const int* idxg = d.idx + (size_t)s * m.idx_total + ioff;
    for (int i = tid; i < S; i += NT) sIdx[i] = idxg[i];
  }
  const f16* pk = reinterpret_cast<const f16*>(d.pkey) + (size_t)s * m.V_cap * 32;
  const bf16* pv = reinterpret_cast<const bf16*>(d.pval) + (size_t)s * m.V_cap * 64;

  // ---- query fragments (B operand of S^T = K . Q^T), pre-scaled by scale*log2(e)
  const bf16* qrow = reinterpret_cast<const bf16*>(src.q) + ((size_t)s * src.n_call + (size_t)(qp - src.p0)) * 64;
  bf16x8 qf[4];    // window: k-step kk holds dims 16kk + 8h + e (rotated for kk < 2)
  f16x8 qs16[2];   // state: dims 32 + 16kk + 8h + e, fp16, scaled by 2^-qsh
  int qsh = 0;
  {
    alignas(16) bf16 x[4][8];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) copy16(x[kk], qrow + 16 * kk + 8 * h);
    const float* rc = d.rope_cos + qp * 16;
    const float* rsn = d.rope_sin + qp * 16;
    float qmx = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float a = tof(x[0][e]), b = tof(x[1][e]);
      rot(a, b, rc[8 * h + e], rsn[8 * h + e]);
      qf[0][e] = (bf16)(a * c2);
      qf[1][e] = (bf16)(b * c2);
      qf[2][e] = (bf16)(tof(x[2][e]) * c2);
      qf[3][e] = (bf16)(tof(x[3][e]) * c2);
      qmx = fmaxf(qmx, fmaxf(fabsf(tof(x[2][e])), fabsf(tof(x[3][e]))) * c2);
    }
    // fp16 range guard for the state query: exact power-of-two pre-scale
    qmx = fmaxf(qmx, partner_f(qmx));
    if (qmx >= 16384.f) {
      int ex;
      frexpf(qmx, &ex);
      qsh = ex - 14;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      qs16[0][e] = (f16)ldexpf(tof(x[2][e]) * c2, -qsh);
      qs16[1][e] = (f16)ldexpf(tof(x[3][e]) * c2, -qsh);
    }
  }
  const bool wave_qsh = __ballot(qsh != 0) != 0ull;

  // ---- running softmax state: acc comes out of the MFMA as logit*c - mref
  float mref = 0.f, lrun = 0.f;
  bool started = false;
  f32x16 negm = {};
  f32x16 O0 = {}, O1 = {};

  // ---- tile geometry: state tiles first, then window tiles
  const int n_st = (S + 63) >> 6;
  const int64_t lo = cpos - m.W > 0 ? cpos - m.W : 0;
  const int64_t hi = cpos + C < end_pos ? cpos + C : end_pos;
  const int n_wt = (int)((hi - lo + 63) >> 6);
  const int n_tiles = n_st + n_wt;
  const int64_t qlast = min(cpos + 32 * w + 31, end_pos - 1);
  const int64_t qfirst = cpos + 32 * w;
  const bf16* krot = reinterpret_cast<const bf16*>(d.krot) + (size_t)s * m.max_tokens * 32;
  const bf16* kin = reinterpret_cast<const bf16*>(src.k) + (size_t)s * src.n_call * 64;
  const bf16* vin = reinterpret_cast<const bf16*>(src.v) + (size_t)s * src.n_call * 64;
  const bf16* ring_k = reinterpret_cast<const bf16*>(d.ring_k) + (size_t)s * m.R * 64;
  const bf16* ring_v = reinterpret_cast<const bf16*>(d.ring_v) + (size_t)s * m.R * 64;

  // ---- lane-constant LDS offsets
  // K operand: key kb + jl, 16-byte unit 2kk + h, swizzled (swz_wk / swz_sk)
  const int kswz_w = swz_wk(jl), kswz_s = swz_sk(jl);
  // V operand (transposed read): group g = lane/16 supplies keys 4h + (lane%16)/4 and
  // dims 32dt + 16(g%2) + 4(lane%4); unit index swizzled (swz_v)
  int voff[2];
  {
    const int g = lane >> 4, p = lane & 15;
    const int kl = 4 * h + (p >> 2);
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) {
      const int d0 = 32 * dt + 16 * (g & 1) + 4 * (p & 3);
      voff[dt] = kl * 128 + 16 * ((d0 >> 3) ^ swz_v(kl)) + 8 * ((d0 >> 2) & 1);
    }
  }

  // ---- direct global->LDS staging of tile T (each wave a share of the 1 KB
  // transfers).  Addresses are a tile-uniform base plus a small per-lane byte
  // offset (version ids zero-extended), which keeps the per-transfer vector
  // arithmetic to a few 32-bit operations.
  auto issue = [&](int T, uint8_t* K, uint8_t* V) {
    if (T < n_st) {
      const int r0 = T << 6;
      // scalar bases, 32-bit lane offsets (a sequence's pool is far below 4 GB)
      const char* pkb = uniform_ptr(reinterpret_cast<const char*>(pk));
      const char* pvb = uniform_ptr(reinterpret_cast<const char*>(pv));
      for (int i = w; i < 4; i += NW) {           // keys: 16 rows x 64 B per transfer
        const int row = 16 * i + (lane >> 2);
        const uint32_t unit = (uint32_t)((lane & 3) ^ swz_sk(row));
        const int r = min(r0 + row, S - 1);
        const uint32_t off = ((uint32_t)sIdx[r] << 6) + 16u * unit;
        __builtin_amdgcn_global_load_lds(pkb + off, K + 1024 * i, 16, 0, 0);
      }
      for (int i = w; i < 8; i += NW) {           // values: 8 rows x 128 B per transfer
        const int row = 8 * i + (lane >> 3);
        const uint32_t unit = (uint32_t)((lane & 7) ^ swz_v(row));
        const int r = min(r0 + row, S - 1);
        const uint32_t off = ((uint32_t)sIdx[r] << 7) + 16u * unit;
        __builtin_amdgcn_global_load_lds(pvb + off, V + 1024 * i, 16, 0, 0);
      }
    } else {
      const int64_t k0 = lo + ((int64_t)(T - n_st) << 6);
      if (k0 >= src.p0) {
        // every key of the tile is an input of this call (the usual case)
        const int last = (int)min((int64_t)63, hi - 1 - k0);
        const char* kr0 = uniform_ptr(reinterpret_cast<const char*>(krot + k0 * 32));
        const char* ki0 = uniform_ptr(reinterpret_cast<const char*>(kin + (k0 - src.p0) * 64));
        const char* vi0 = uniform_ptr(reinterpret_cast<const char*>(vin + (k0 - src.p0) * 64));
        for (int i = w; i < 8; i += NW) {         // keys and values: 8 keys x 128 B per transfer
          const int key = 8 * i + (lane >> 3);
          const uint32_t unit = (uint32_t)((lane & 7) ^ swz_wk(key));
          const uint32_t vunit = (uint32_t)((lane & 7) ^ swz_v(key));
          const uint32_t kc = (uint32_t)min(key, last);
          const char* ks = unit < 4 ? kr0 + (kc * 64u + 16u * unit) : ki0 + (kc * 128u + 16u * unit);
          const char* vs = vi0 + (kc * 128u + 16u * vunit);
          __builtin_amdgcn_global_load_lds(ks, K + 1024 * i, 16, 0, 0);
          __builtin_amdgcn_global_load_lds(vs, V + 1024 * i, 16, 0, 0);
        }
      } else {
        for (int i = w; i < 8; i += NW) {
          const int key = 8 * i + (lane >> 3);
          const int unit = (lane & 7) ^ swz_wk(key);
          const int vunit = (lane & 7) ^ swz_v(key);
          const int64_t pos = min(k0 + key, hi - 1);
          const bf16* ks;
          const bf16* vs;
          if (pos >= src.p0) {
            const size_t r = (size_t)(pos - src.p0) * 64;
            ks = unit < 4 ? krot + pos * 32 + 8 * unit : kin + r + 8 * unit;
            vs = vin + r + 8 * vunit;
          } else {
            const size_t r = (size_t)(pos % m.R) * 64;   // ring keys are stored rotated
            ks = ring_k + r + 8 * unit;
            vs = ring_v + r + 8 * vunit;
          }
          __builtin_amdgcn_global_load_lds(ks, K + 1024 * i, 16, 0, 0);
          __builtin_amdgcn_global_load_lds(vs, V + 1024 * i, 16, 0, 0);
        }
      }
    }
  };

  // ---- online softmax of one 64-key tile (two 32-key subtiles, the second
  // optional): one maximum, one rescale decision, p packed to bf16 and the row
  // sum taken from the packed p
  auto softmax = [&](f32x16& a0, f32x16& a1, bool two, bf16x8 (&pf)[4]) {
    float mx = fmaxf(a0[0], a0[1]);
#pragma unroll
    for (int r = 2; r < 16; r += 2) mx = fmaxf(fmaxf(mx, a0[r]), a0[r + 1]);
    if (two) {
#pragma unroll
      for (int r = 0; r < 16; r += 2) mx = fmaxf(fmaxf(mx, a1[r]), a1[r + 1]);
    }
    mx = fmaxf(mx, partner_f(mx));
    if ((!started && mx != -kInf) || mx > kTau) {
      if (started) {
        const float alpha = exp2_fast(-mx);
        lrun *= alpha;
#pragma unroll
        for (int r = 0; r < 16; ++r) { O0[r] *= alpha; O1[r] *= alpha; }
      }
      mref += mx;
#pragma unroll
      for (int r = 0; r < 16; ++r) { a0[r] -= mx; a1[r] -= mx; negm[r] = -mref; }
      started = true;
    }
    const bf16x2 one = {(bf16)1.f, (bf16)1.f};
    float ls = lrun;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pf[0][e] = (bf16)exp2_fast(a0[e]);
      pf[1][e] = (bf16)exp2_fast(a0[8 + e]);
    }
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      ls = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pf[0][e], pf[0][e + 1]}, one, ls, false);
      ls = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pf[1][e], pf[1][e + 1]}, one, ls, false);
    }
    if (two) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pf[2][e] = (bf16)exp2_fast(a1[e]);
        pf[3][e] = (bf16)exp2_fast(a1[8 + e]);
      }
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        ls = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pf[2][e], pf[2][e + 1]}, one, ls, false);
        ls = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pf[3][e], pf[3][e + 1]}, one, ls, false);
      }
    }
    lrun = ls;
  };
  // O^T += V^T . P^T over the 32 keys [kb, kb + 32) of the staged tile.  The
  // V^T fragment of (dt, b) = (0, 0) can be read ahead (vfrag) so that its
  // LDS latency passes during the softmax.
  auto vfrag = [&](const uint8_t* V, int kb, int dt, int b) {
    const uint8_t* base = V + (kb + 16 * b) * 128 + voff[dt];
    const bf16x4 lo4 = ds_read_tr(base);
    const bf16x4 hi4 = ds_read_tr(base + 8 * 128);
    return bf16x8{lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
  };
  auto pv_acc = [&](const uint8_t* V, int kb, const bf16x8& pf0, const bf16x8& pf1, const bf16x8& v00) {
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) {
      f32x16& O = dt ? O1 : O0;
#pragma unroll
      for (int b = 0; b < 2; ++b) O = mfma_bf16(dt == 0 && b == 0 ? v00 : vfrag(V, kb, dt, b), b ? pf1 : pf0, O);
    }
  };
  // masks keys at offsets >= lim of a 32-key subtile (this lane's rows 8(r/4) + 4h + r%4)
  auto mask = [&](f32x16& acc, int lim) {
    if (lim < 32) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (8 * (r >> 2) + 4 * h + (r & 3) >= lim) acc[r] = -kInf;
    }
  };
  auto compute = [&](int T, const uint8_t* K, const uint8_t* V) {
    f32x16 a0, a1;
    bool two;
    if (T < n_st) {
      const int r0 = T << 6;
      two = r0 + 32 < S;
      auto qk = [&](int kb, f32x16& acc) {
        const uint8_t* kr = K + (kb + jl) * 64;
        const f16x8 k0v = *reinterpret_cast<const f16x8*>(kr + 16 * (h ^ kswz_s));
        const f16x8 k1v = *reinterpret_cast<const f16x8*>(kr + 16 * ((2 + h) ^ kswz_s));
        if (!wave_qsh) {
          acc = mfma_f16(k0v, qs16[0], negm);
          acc = mfma_f16(k1v, qs16[1], acc);
        } else {
          acc = mfma_f16(k0v, qs16[0], f32x16{});
          acc = mfma_f16(k1v, qs16[1], acc);
          const float sc = ldexpf(1.f, qsh);
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[r] = acc[r] * sc - mref;
        }
      };
      qk(0, a0);
      mask(a0, S - r0);
      if (two) {
        qk(32, a1);
        mask(a1, S - r0 - 32);
      }
    } else {
      const int64_t k0 = lo + ((int64_t)(T - n_st) << 6);
      if (k0 > qlast) return;   // every key of the tile is after this wave's queries
      two = k0 + 32 < hi && k0 + 32 <= qlast;
      auto qk = [&](int kb, f32x16& acc) {
        const uint8_t* kr = K + (kb + jl) * 128;
        acc = mfma_bf16(*reinterpret_cast<const bf16x8*>(kr + 16 * (h ^ kswz_w)), qf[0], negm);
#pragma unroll
        for (int kk = 1; kk < 4; ++kk)
          acc = mfma_bf16(*reinterpret_cast<const bf16x8*>(kr + 16 * ((2 * kk + h) ^ kswz_w)), qf[kk], acc);
        const int64_t ks = k0 + kb;
        // key ks + off is valid for this lane's query iff off < lim
        // (32-bit per lane: the query's offset 32 w + jl in the chunk plus the
        // uniform distance from the key tile to the chunk start)
        if (ks + 31 >= hi || ks + 31 > qfirst) mask(acc, min((int)(hi - ks), (int)(cpos - ks) + 32 * w + jl + 1));
      };
      qk(0, a0);
      if (two) qk(32, a1);
    }
    const bf16x8 v00 = vfrag(V, 0, 0, 0);   // in flight during the softmax
    bf16x8 pf[4];
    softmax(a0, a1, two, pf);
    pv_acc(V, 0, pf[0], pf[1], v00);
    if (two) pv_acc(V, 32, pf[2], pf[3], vfrag(V, 32, 0, 0));
  };

  // ---- two-stage pipeline; each barrier also waits for the wave's own transfers
  __syncthreads();   // version ids in LDS
  if (n_tiles > 0) issue(0, sK0, sV0);
  for (int T = 0; T < n_tiles; T += 2) {
    dma_barrier();   // tile T in stage 0; stage 1 free
    if (T + 1 < n_tiles) issue(T + 1, sK1, sV1);
    compute(T, sK0, sV0);
    if (T + 1 >= n_tiles) break;
    dma_barrier();   // tile T+1 in stage 1; stage 0 free
    if (T + 2 < n_tiles) issue(T + 2, sK0, sV0);
    compute(T + 1, sK1, sV1);
  }

  // ---- normalise and store: lane holds dims 8*(r/4) + 4h + r%4 of its query
  const float lt = lrun + partner_f(lrun);
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;
  if (qvalid) {
    bf16* orow = out + ((size_t)s * src.n_call + (size_t)(qpos - src.p0)) * 64;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) {
      const f32x16& O = dt ? O1 : O0;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        alignas(8) bf16 vals[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) vals[e] = (bf16)(O[4 * g4 + e] * inv);
        *reinterpret_cast<uint2*>(orow + 32 * dt + 8 * g4 + 4 * h) = *reinterpret_cast<const uint2*>(vals);
      }
    }
  }
}

// RoPE prep for the DMA attention: rotary dims [0, 32) of every key of the call,
// rotated at its absolute position, into krot[BH][max_tokens][32] (bf16).
__global__ void rope_keys_kernel(Dims m, Dev d, Src src) {
  const int64_t n = (int64_t)m.BH * src.n_call * 2;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int hh = (int)(i & 1);
    const int64_t tok = i >> 1;
    const int s = (int)(tok / src.n_call);
    int64_t p0 = src.p0;
    if (src.seq) {
      const int64_t* sr = src.seq + (size_t)s * kSeqFields;
      if (tok % src.n_call >= sr[kSeqN]) continue;   // padding past this sequence's tokens
      p0 = sr[kSeqP0];
    }
    const int64_t pos = p0 + tok % src.n_call;
    const bf16* kr = reinterpret_cast<const bf16*>(src.k) + (size_t)tok * 64;
    alignas(16) bf16 x[8], y[8];
    copy16(x, kr + 8 * hh);
    copy16(y, kr + 16 + 8 * hh);
    const float* rc = d.rope_cos + pos * 16 + 8 * hh;
    const float* rs = d.rope_sin + pos * 16 + 8 * hh;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float a = tof(x[e]), b = tof(y[e]);
      rot(a, b, rc[e], rs[e]);
      x[e] = (bf16)a;
      y[e] = (bf16)b;
    }
    bf16* dst = reinterpret_cast<bf16*>(d.krot) + ((size_t)s * m.max_tokens + (size_t)pos) * 32;
    copy16(dst + 8 * hh, x);
    copy16(dst + 16 + 8 * hh, y);
  }
}

// =====================================================================
// Ring maintenance: the last W + C positions (rotated keys, values, gate
// logits) are kept so that decode steps and later prefill calls can see the
// window and absorb the chunk that leaves it.
// =====================================================================
template <typename T>
__global__ __launch_bounds__(256) void ring_fill_kernel(Dims m, Dev d, Src src, int64_t from, int64_t to) {
  // four tokens per workgroup, one lane per dimension
  const int s = blockIdx.y;
  if (src.seq) {
    const int64_t* sr = src.seq + (size_t)s * kSeqFields;
    src.p0 = sr[kSeqP0];
    from = sr[kSeqFrom];
    to = sr[kSeqTo];
  }
  const int64_t pos = from + (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (pos >= to) return;
  const int dd = threadIdx.x & 63;
  T* rk = reinterpret_cast<T*>(d.ring_k) + (size_t)s * m.R * 64;
  T* rv = reinterpret_cast<T*>(d.ring_v) + (size_t)s * m.R * 64;
  float* rl = d.ring_l + (size_t)s * m.R;
  const size_t r = (size_t)s * src.n_call + (size_t)(pos - src.p0);
  const T* kr = reinterpret_cast<const T*>(src.k) + r * 64;
  const T* vr = reinterpret_cast<const T*>(src.v) + r * 64;
  float x = tof(kr[dd]);
  if (dd < 32) {
    const int jf = dd & 15;
    const float cs = d.rope_cos[pos * 16 + jf], sn = d.rope_sin[pos * 16 + jf];
    x = dd < 16 ? x * cs - tof(kr[dd + 16]) * sn : x * cs + tof(kr[dd - 16]) * sn;
  }
  const size_t slot = (size_t)(pos % m.R);
  rk[slot * 64 + dd] = fromf<T>(x);
  rv[slot * 64 + dd] = vr[dd];
  if (dd == 0) rl[slot] = src.l[r];
}

// =====================================================================
// Decode ([KVM abstract]: per-token cost independent of the context length;
// [KVM summary, Core mechanisms 4]): one workgroup of eight waves per
// sequence.  The new token's rotated key, value and gate logit go to ring slot
// t % R; query t attends over the state rows (unrotated q against the
// read-form keys, values rho * u) and the window [lo, t] (rotated q against
// rotated keys) with one softmax.
// The step is bound by reading the state rows and the window once, so the
// kernel is laid out for bytes in flight: the keys and values are read in two
// separate passes over blocks of up to kDecBlock logits.  Pass 1 computes the
// block's logits into LDS (a few lanes per key, 16 bytes each, several keys
// per lane in flight, no dependence between keys); the block's maximum then
// gives exact weights; pass 2 streams the values and accumulates
// p * v (again several rows per lane in flight, no running-maximum chain).
// A state larger than one block rescales the accumulators between blocks.
// State rows are read with non-temporal loads: each is used once per step.
// =====================================================================
constexpr int kDecWaves = 4;
constexpr int kDecBlock = 2048;   // logits per block (8 KB of LDS)
constexpr int kDecUnroll = 2;     // keys or value rows per lane in each batch (two batches in flight)

__device__ __forceinline__ u32x4 ld_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// 16 bytes as floats: 8 bf16, 8 fp16 or 4 f32 (the first 16 / sizeof(E) entries of f)
template <typename E>
__device__ __forceinline__ void unpack16(const u32x4& x, float* f) {
  if constexpr (sizeof(E) == 4) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(x[i]);
  } else if constexpr (std::is_same<E, bf16>::value) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(x[i] << 16);
      f[2 * i + 1] = __uint_as_float(x[i] & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = (float)__builtin_bit_cast(f16, (uint16_t)(x[i] & 0xFFFFu));
      f[2 * i + 1] = (float)__builtin_bit_cast(f16, (uint16_t)(x[i] >> 16));
    }
  }
}

// maximum over the wave, every lane getting it
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, xor_lane<1>(x));
  x = fmaxf(x, xor_lane<2>(x));
  x = fmaxf(x, dpp_mov<0x141>(x));
  x = fmaxf(x, dpp_mov<0x140>(x));
  float a, b;
  row_pair(x, a, b);
  x = fmaxf(a, b);
  half_pair(x, a, b);
  return fmaxf(a, b);
}

// sum over aligned groups of G lanes (G a power of two <= 16)
template <int G>
__device__ __forceinline__ float dec_group_sum(float x) {
  return group_sum<G>(x);
}

template <typename T>
__global__ __launch_bounds__(64 * kDecWaves) void dec_kernel(Dims m, Dev d, const T* q, const T* kin, const T* vin,
                                                            const float* lin, T* out, int64_t t, int S,
                                                            int64_t lo, const int64_t* seq) {
  using RT = typename Rd<T>::type;
  constexpr int NT = 64 * kDecWaves;
  constexpr int KE = 16 / (int)sizeof(RT);   // state-key dims per lane (of 32)
  constexpr int KL = 32 / KE;                // lanes per state key
  constexpr int VE = 16 / (int)sizeof(T);    // value (and window-key) dims per lane (of 64)
  constexpr int VL = 64 / VE;                // lanes per value row / window key
  constexpr int U = kDecUnroll;
  __shared__ float sq[64], sqr[64], skt[64], svt[64];
  __shared__ float sL[kDecBlock];
  __shared__ float red[kDecWaves];
  __shared__ float red_o[kDecWaves][64];
  const int s = blockIdx.x;
  if (seq) {   // this sequence's own position; its window and state follow from it
    const int64_t* sr = seq + (size_t)s * kSeqFields;
    if (!sr[kSeqActive]) return;
    t = sr[kSeqPos];
    const int64_t c = t / m.C;
    lo = c * m.C - m.W > 0 ? c * m.C - m.W : 0;
    const int64_t absorbed = c - m.W / m.C > 0 ? c - m.W / m.C : 0;   // chunks absorbed once t is consumed
    S = 0;
    if (absorbed > 0) {
      const int4 sc = d.sched[absorbed - 1];
      S = sc.x + sc.y + sc.z;
    }
  }
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const float sl2 = m.scale * kLog2e;
  if (tid < 64) {
    // query (scaled into log2 units) and the new token; RoPE on dims [0, 32)
    const T* qr = q + (size_t)s * 64;
    const T* kr = kin + (size_t)s * 64;
    float x = tof(qr[tid]), y = x, kx = tof(kr[tid]);
    if (tid < 32) {
      const int jf = tid & 15;
      const float cs = d.rope_cos[t * 16 + jf], sn = d.rope_sin[t * 16 + jf];
      y = tid < 16 ? x * cs - tof(qr[tid + 16]) * sn : x * cs + tof(qr[tid - 16]) * sn;
      kx = tid < 16 ? kx * cs - tof(kr[tid + 16]) * sn : kx * cs + tof(kr[tid - 16]) * sn;
    }
    const T kq = fromf<T>(kx);
    const T vv = vin[(size_t)s * 64 + tid];
    sq[tid] = x * sl2;
    sqr[tid] = y * sl2;
    skt[tid] = tof(kq);
    svt[tid] = tof(vv);
    const size_t slot = (size_t)s * m.R + (size_t)(t % m.R);
    reinterpret_cast<T*>(d.ring_k)[slot * 64 + tid] = kq;
    reinterpret_cast<T*>(d.ring_v)[slot * 64 + tid] = vv;
    if (tid == 0) d.ring_l[slot] = lin[s];
  }
  __syncthreads();

  const char* kr = reinterpret_cast<const char*>(d.kread) + (size_t)s * m.S_cap * 32 * sizeof(RT);
  const char* vr = reinterpret_cast<const char*>(d.vread) + (size_t)s * m.S_cap * 64 * sizeof(T);
  const char* rk = reinterpret_cast<const char*>(d.ring_k) + (size_t)s * m.R * 64 * sizeof(T);
  const char* rv = reinterpret_cast<const char*>(d.ring_v) + (size_t)s * m.R * 64 * sizeof(T);
  const int nw = (int)(t - lo + 1);          // window keys, position t last
  const int total = S + nw;
  const int ksub = lane % KL, kgrp = lane / KL;   // pass 1, state keys
  const int vsub = lane % VL, vgrp = lane / VL;   // pass 1 window keys and pass 2
  float qs[KE], qw[VE];
#pragma unroll
  for (int i = 0; i < KE; ++i) qs[i] = sq[32 + KE * ksub + i];
#pragma unroll
  for (int i = 0; i < VE; ++i) qw[i] = sqr[VE * vsub + i];

  float M = -kInf, lsum = 0.f;
  float o[VE];
#pragma unroll
  for (int i = 0; i < VE; ++i) o[i] = 0.f;

  for (int b0 = 0; b0 < total; b0 += kDecBlock) {
    const int b1 = min(total, b0 + kDecBlock);
    // ---- pass 1: logits of [b0, b1) into sL
    {
      // software-pipelined: the next batch of keys is requested before this one is used
      const int e1 = min(b1, S);
      constexpr int PER = 64 / KL * kDecWaves;   // state keys per round of the workgroup
      auto load = [&](u32x4 (&x)[U], int r0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int r = max(min(r0 + u * PER, e1 - 1), 0);
          x[u] = ld_nt(kr + (size_t)r * 32 * sizeof(RT) + 16 * ksub);
        }
      };
      int r0 = b0 + w * (64 / KL) + kgrp;
      u32x4 x[U];
      if (r0 < e1) load(x, r0);
      for (; r0 < e1; r0 += PER * U) {
        u32x4 xn[U];
        if (r0 + PER * U < e1) load(xn, r0 + PER * U);
#pragma unroll
        for (int u = 0; u < U; ++u) {
          float f[8];
          unpack16<RT>(x[u], f);
          float dot = 0.f;
#pragma unroll
          for (int i = 0; i < KE; ++i) dot = fmaf(qs[i], f[i], dot);
          dot = dec_group_sum<KL>(dot);
          const int r = r0 + u * PER;
          if (ksub == 0 && r < e1) sL[r - b0] = dot;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) x[u] = xn[u];
      }
    }
    {
      const int e0 = max(b0, S);
      constexpr int PER = 64 / VL * kDecWaves;   // window keys per round
      for (int i0 = e0 - S + w * (64 / VL) + vgrp; i0 + S < b1; i0 += PER * U) {
        u32x4 x[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int i = min(i0 + u * PER, b1 - S - 1);
          const int64_t pos = lo + i;
          x[u] = pos == t ? u32x4{0u, 0u, 0u, 0u}
                          : ld16(rk + ((size_t)(pos % m.R) * 64 + VE * vsub) * sizeof(T));
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int i = i0 + u * PER;
          float f[8];
          unpack16<T>(x[u], f);
          if (lo + i == t) {
#pragma unroll
            for (int k = 0; k < VE; ++k) f[k] = skt[VE * vsub + k];
          }
          float dot = 0.f;
#pragma unroll
          for (int k = 0; k < VE; ++k) dot = fmaf(qw[k], f[k], dot);
          dot = dec_group_sum<VL>(dot);
          if (vsub == 0 && i + S < b1) sL[i + S - b0] = dot;
        }
      }
    }
    // the first batch of pass 2's values is requested now, so that it is in
    // flight while the block's maximum and weights are formed
    const int ve1 = min(b1, S);
    constexpr int VPER = 64 / VL * kDecWaves;   // value rows per round of the workgroup
    auto vload = [&](u32x4 (&x)[U], int r0) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int r = max(min(r0 + u * VPER, ve1 - 1), 0);
        x[u] = ld_nt(vr + ((size_t)r * 64 + VE * vsub) * sizeof(T));
      }
    };
    int vr0 = b0 + w * (64 / VL) + vgrp;
    u32x4 vx[U];
    if (vr0 < ve1) vload(vx, vr0);
    __syncthreads();
    // ---- the block's maximum, then exact weights in place
    float mx = -kInf;
    for (int i = tid; i < b1 - b0; i += NT) mx = fmaxf(mx, sL[i]);
    mx = wave_max(mx);
    if (lane == 0) red[w] = mx;
    __syncthreads();
    mx = red[0];
#pragma unroll
    for (int ww = 1; ww < kDecWaves; ++ww) mx = fmaxf(mx, red[ww]);
    const float Mn = fmaxf(M, mx);
    const float sc = M == -kInf ? 0.f : exp2_fast(M - Mn);
    M = Mn;
    lsum *= sc;
#pragma unroll
    for (int i = 0; i < VE; ++i) o[i] *= sc;
    for (int i = tid; i < b1 - b0; i += NT) {
      const float p = exp2_fast(sL[i] - M);
      sL[i] = p;
      lsum += p;
    }
    __syncthreads();
    // ---- pass 2: values of [b0, b1)
    for (; vr0 < ve1; vr0 += VPER * U) {
      u32x4 xn[U];
      if (vr0 + VPER * U < ve1) vload(xn, vr0 + VPER * U);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int r = vr0 + u * VPER;
        const float p = r < ve1 ? sL[r - b0] : 0.f;
        float f[8];
        unpack16<T>(vx[u], f);
#pragma unroll
        for (int k = 0; k < VE; ++k) o[k] = fmaf(p, f[k], o[k]);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) vx[u] = xn[u];
    }
    {
      const int e0 = max(b0, S);
      constexpr int PER = 64 / VL * kDecWaves;
      for (int i0 = e0 - S + w * (64 / VL) + vgrp; i0 + S < b1; i0 += PER * U) {
        u32x4 x[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int i = min(i0 + u * PER, b1 - S - 1);
          const int64_t pos = lo + i;
          x[u] = pos == t ? u32x4{0u, 0u, 0u, 0u}
                          : ld16(rv + ((size_t)(pos % m.R) * 64 + VE * vsub) * sizeof(T));
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int i = i0 + u * PER;
          const float p = i + S < b1 ? sL[i + S - b0] : 0.f;
          float f[8];
          unpack16<T>(x[u], f);
          if (lo + i == t) {
#pragma unroll
            for (int k = 0; k < VE; ++k) f[k] = svt[VE * vsub + k];
          }
#pragma unroll
          for (int k = 0; k < VE; ++k) o[k] = fmaf(p, f[k], o[k]);
        }
      }
    }
    __syncthreads();   // sL is rewritten by the next block
  }
  // ---- combine: lane groups of the wave (same dims), then the waves; the row sum over all threads
#pragma unroll
  for (int k = 0; k < VE; ++k) {
    if constexpr (VL == 8) o[k] += dpp_mov<0x128>(o[k]);   // row_ror:8, the group 8 lanes away
    float a, b;
    row_pair(o[k], a, b);
    o[k] = a + b;
    half_pair(o[k], a, b);
    o[k] = a + b;
  }
  lsum = group_sum<64>(lsum);
  if (lane < VL) {
#pragma unroll
    for (int k = 0; k < VE; ++k) red_o[w][VE * lane + k] = o[k];
  }
  if (lane == 0) red[w] = lsum;
  __syncthreads();
  if (tid < 64) {
    float Ls = 0.f, Ov = 0.f;
#pragma unroll
    for (int ww = 0; ww < kDecWaves; ++ww) {
      Ls += red[ww];
      Ov += red_o[ww][tid];
    }
    out[(size_t)s * 64 + tid] = fromf<T>(Ls > 0.f ? Ov / Ls : 0.f);
  }
}

template <typename T>
__global__ void snapshot_gather_kernel(Dims m, Dev d, int rows, int64_t ioff, int stride,
                                       typename Rd<T>::type* key_out, T* val_out, float* rho_out, int* count_out) {
  using RT = typename Rd<T>::type;
  const int s = blockIdx.x;
  const int* idxl = d.idx + (size_t)s * m.idx_total + ioff;
  const RT* pk = reinterpret_cast<const RT*>(d.pkey) + (size_t)s * m.V_cap * 32;
  const T* pv = reinterpret_cast<const T*>(d.pval) + (size_t)s * m.V_cap * 64;
  const float* pr = d.prho + (size_t)s * m.V_cap;
  const int* pc = d.pcount + (size_t)s * m.V_cap;
  for (int64_t i = threadIdx.x; i < (int64_t)rows * 98; i += blockDim.x) {
    const int r = (int)(i / 98), dd = (int)(i % 98);
    const int64_t ver = idxl[r];
    const size_t o = (size_t)s * stride + r;
    if (dd < 32) {
      if (key_out) key_out[o * 32 + dd] = pk[ver * 32 + dd];
    } else if (dd < 96) {
      if (val_out) val_out[o * 64 + dd - 32] = pv[ver * 64 + dd - 32];
    } else if (dd == 96) {
      if (rho_out) rho_out[o] = pr[ver];
    } else if (count_out) {
      count_out[o] = pc[ver];
    }
  }
}

// State load: one workgroup per sequence, four lanes per row (the lane layout of
// the scan's row update, so that row_derive gives the same bits).  Version id of
// row r = r; the index list of the last absorbed chunk names them.
template <typename T>
__global__ __launch_bounds__(256) void state_load_kernel(Dims m, Dev d, int rows, int64_t ioff) {
  using RT = typename Rd<T>::type;
  const int s = blockIdx.x;
  const int sub = threadIdx.x & 3;
  const float* key_sum = d.key_sum + (size_t)s * m.S_cap * 32;
  const float* val_sum = d.val_sum + (size_t)s * m.S_cap * 64;
  const int* count = d.count + (size_t)s * m.S_cap;
  const float* rho = d.rho + (size_t)s * m.S_cap;
  char* unit = reinterpret_cast<char*>(d.unit) + (size_t)s * m.S_cap * 128;
  RT* kread = reinterpret_cast<RT*>(d.kread) + (size_t)s * m.S_cap * 32;
  T* vread = reinterpret_cast<T*>(d.vread) + (size_t)s * m.S_cap * 64;
  RT* pkey = reinterpret_cast<RT*>(d.pkey) + (size_t)s * m.V_cap * 32;
  T* pval = reinterpret_cast<T*>(d.pval) + (size_t)s * m.V_cap * 64;
  float* prho = d.prho + (size_t)s * m.V_cap;
  int* pcount = d.pcount + (size_t)s * m.V_cap;
  for (int r = threadIdx.x >> 2; r < rows; r += blockDim.x >> 2) {
    RowRegs rr;
    row_load(rr, key_sum, val_sum, count, rho, r, sub);
    float K[8], V[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      K[i] = rr.k[0][i];
      K[4 + i] = rr.k[1][i];
#pragma unroll
      for (int q = 0; q < 4; ++q) V[4 * q + i] = rr.v[q][i];
    }
    float rs, vsc;
    row_derive<T>(K, V, rr.n, rr.rh, sub, m, unit + (size_t)r * 128, nullptr, kread + (size_t)r * 32,
                  vread + (size_t)r * 64, pkey + (size_t)r * 32, pval + (size_t)r * 64, rs, vsc);
    if (sub == 0) {
      prho[r] = rr.rh;
      pcount[r] = rr.n;
      d.pnorm[(size_t)s * m.V_cap + r] = make_float2(rs, vsc);
      if (ioff >= 0) d.idx[(size_t)s * m.idx_total + ioff + r] = r;
    }
  }
  if (threadIdx.x == 0) d.nver[s] = rows;
}

// One sequence back to an empty state: its version counter and scan exchange
// records (tag 0) cleared, its trace marked "not absorbed".
__global__ void seq_reset_kernel(Dims m, Dev d, int s) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n = (int64_t)gridDim.x * blockDim.x;
  const int64_t xw = (int64_t)2 * m.P * m.C;
  uint2* xb = d.xbuf + (size_t)s * xw;
  for (int64_t k = i; k < xw; k += n) xb[k] = make_uint2(0u, 0u);
  if (m.trace)
    for (int64_t k = i; k < m.max_tokens; k += n) {
      d.tslot[(size_t)s * m.max_tokens + k] = -1;
      d.tkind[(size_t)s * m.max_tokens + k] = 0xFF;
    }
  if (i == 0) d.nver[s] = 0;
}

// Schedule table of a workspace in the static scratch (one thread: at most a few
// thousand chunks), with the host's rules: sinks first, then
// m_j = min(max(capacity((j + 1) C) - rows, 0), candidates), capacity =
// max_slots (fixed), ceil(alpha sqrt(T)) (sqrt, as the integer ceil-sqrt of
// alpha^2 T) or the smaller of the two (saturating).  Every other thread
// zeroes the version counters and the scan's exchange buffers.
__global__ void noalloc_init_kernel(SchedParams sp, int4* sched, int* nver, int bh, uint2* xbuf, int64_t xwords,
                                    int* xerr) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n = (int64_t)gridDim.x * blockDim.x;
  for (int64_t k = i; k < xwords; k += n) xbuf[k] = make_uint2(0u, 0u);
  for (int64_t k = i; k < bh; k += n) nver[k] = 0;
  if (i != 0) return;
  *xerr = 0;
  int64_t rows = 0, nsink = 0, idx_off = 0;
  for (int j = 0; j < sp.J; ++j) {
    int64_t cand = sp.C;
    const int64_t sk = min((int64_t)sp.ns - nsink, cand);
    const int64_t before = rows;
    nsink += sk;
    rows += sk;
    cand -= sk;
    const uint64_t T = (uint64_t)(j + 1) * (uint64_t)sp.C;
    int64_t cap = sp.max_slots;
    if (sp.sched != 0) {
      const uint64_t x = (uint64_t)sp.alpha * (uint64_t)sp.alpha * T;
      uint64_t r = (uint64_t)sqrt((double)x);
      while (r > 0 && r * r > x) --r;
      while ((r + 1) * (r + 1) <= x) ++r;
      const int64_t cs = (int64_t)(r * r == x ? r : r + 1);
      cap = sp.sched == 1 ? cs : min(cs, (int64_t)sp.max_slots);
    }
    int64_t m = cap - rows;
    if (m < 0) m = 0;
    if (m > cand) m = cand;
    rows += m;
    sched[j] = make_int4((int)sk, (int)m, (int)before, (int)idx_off);
    idx_off += rows;
  }
}

template <typename T>
hipError_t scan_dispatch(const Dims& m, const Dev& d, const Src& src, int jb, int je, hipStream_t st) {
  const bool part = m.P > 1;
  switch (m.C) {
    case 32:
      if (part) scan_kernel<T, 32, true><<<m.BH * m.P, ScanGeom<32>::NT, 0, st>>>(m, d, src, d.sched, jb, je);
      else scan_kernel<T, 32, false><<<m.BH, ScanGeom<32>::NT, 0, st>>>(m, d, src, d.sched, jb, je);
      break;
    case 64:
      if (part) scan_kernel<T, 64, true><<<m.BH * m.P, ScanGeom<64>::NT, 0, st>>>(m, d, src, d.sched, jb, je);
      else scan_kernel<T, 64, false><<<m.BH, ScanGeom<64>::NT, 0, st>>>(m, d, src, d.sched, jb, je);
      break;
    case 128:
      if (part) scan_kernel<T, 128, true><<<m.BH * m.P, ScanGeom<128>::NT, 0, st>>>(m, d, src, d.sched, jb, je);
      else scan_kernel<T, 128, false><<<m.BH, ScanGeom<128>::NT, 0, st>>>(m, d, src, d.sched, jb, je);
      break;
    case 256:
      if (part) scan_kernel<T, 256, true><<<m.BH * m.P, ScanGeom<256>::NT, 0, st>>>(m, d, src, d.sched, jb, je);
      else scan_kernel<T, 256, false><<<m.BH, ScanGeom<256>::NT, 0, st>>>(m, d, src, d.sched, jb, je);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t attn_dispatch(const Dims& m, const Dev& d, const Src& src, int64_t cb, int nq, int64_t end, void* out,
                         int s_max, hipStream_t st) {
  const dim3 grid((unsigned)(m.BH * nq));
  T* o = reinterpret_cast<T*>(out);
  const bool dma = Is<T>::bf && d.krot != nullptr && s_max <= kDmaIdxCap;
  const size_t idx_bytes = (size_t)(s_max > 0 ? s_max : 1) * 4;
  switch (m.C) {
    case 32: attn_kernel<T, 1><<<grid, 64, 0, st>>>(m, d, src, cb, nq, end, o); break;
    case 64: attn_kernel<T, 2><<<grid, 128, 0, st>>>(m, d, src, cb, nq, end, o); break;
    case 128:
      if constexpr (Is<T>::bf) {
        if (dma) attn_dma_kernel<4><<<grid, 256, idx_bytes, st>>>(m, d, src, cb, nq, end, o);
        else attn_bf16_kernel<4><<<grid, 256, 0, st>>>(m, d, src, cb, nq, end, o);
      } else {
        attn_kernel<T, 4><<<grid, 256, 0, st>>>(m, d, src, cb, nq, end, o);
      }
      break;
    case 256:
      if constexpr (Is<T>::bf) {
        if (dma) attn_dma_kernel<8><<<grid, 512, idx_bytes, st>>>(m, d, src, cb, nq, end, o);
        else attn_bf16_kernel<8><<<grid, 512, 0, st>>>(m, d, src, cb, nq, end, o);
      } else {
        attn_kernel<T, 8><<<grid, 512, 0, st>>>(m, d, src, cb, nq, end, o);
      }
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_init(const Dims& m, const Dev& d, double theta, hipStream_t st) {
  const int64_t n = m.max_tokens * 16;
  rope_table_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(d.rope_cos, d.rope_sin, m.max_tokens, theta);
  return hipGetLastError();
}

hipError_t launch_seq_reset(const Dims& m, const Dev& d, int s, hipStream_t st) {
  seq_reset_kernel<<<64, 256, 0, st>>>(m, d, s);
  return hipGetLastError();
}

hipError_t launch_noalloc_init(const Dims& m, const Dev& d, const SchedParams& sp, double theta, hipStream_t st) {
  hipError_t e = launch_init(m, d, theta, st);
  if (e != hipSuccess) return e;
  const int64_t xwords = (int64_t)m.BH * 2 * m.P * m.C;
  const int64_t work = xwords > m.BH ? xwords : m.BH;
  const unsigned blocks = (unsigned)std::min<int64_t>((work + 255) / 256, 1024);
  noalloc_init_kernel<<<blocks, 256, 0, st>>>(sp, d.sched, d.nver, m.BH, d.xbuf, xwords, d.xerr);
  return hipGetLastError();
}

hipError_t scratch_address(void** out) {
  // One lookup per device, with that device current: each GPU holds its own
  // copy of the array at its own address.  The name of the array is a host-side
  // stand-in and is never passed to a kernel or a copy.
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

int scan_lds_rows(int C, bool is_bf16) {
  if (!is_bf16) return 0;
  switch (C) {
    case 32: return ScanUnitLds<bf16, 32, true>::NL;
    case 64: return ScanUnitLds<bf16, 64, true>::NL;
    case 128: return ScanUnitLds<bf16, 128, true>::NL;
    case 256: return ScanUnitLds<bf16, 256, true>::NL;
    default: return 0;
  }
}

hipError_t launch_scan(const Dims& m, const Dev& d, const Src& src, int jb, int je, hipStream_t st) {
  if (je <= jb) return hipSuccess;
  return m.bf16 ? scan_dispatch<bf16>(m, d, src, jb, je, st) : scan_dispatch<float>(m, d, src, jb, je, st);
}

hipError_t launch_attn(const Dims& m, const Dev& d, const Src& src, int64_t cb, int nq, int64_t end, void* out,
                       int s_max, hipStream_t st) {
  if (nq <= 0) return hipSuccess;
  return m.bf16 ? attn_dispatch<bf16>(m, d, src, cb, nq, end, out, s_max, st)
                : attn_dispatch<float>(m, d, src, cb, nq, end, out, s_max, st);
}

hipError_t launch_rope_keys(const Dims& m, const Dev& d, const Src& src, hipStream_t st) {
  if (!d.krot || src.n_call <= 0) return hipSuccess;
  const int64_t n = (int64_t)m.BH * src.n_call * 2;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 65536);
  rope_keys_kernel<<<(unsigned)blocks, 256, 0, st>>>(m, d, src);
  return hipGetLastError();
}

hipError_t launch_ring_fill(const Dims& m, const Dev& d, const Src& src, int64_t from, int64_t to, hipStream_t st) {
  if (to <= from) return hipSuccess;
  const dim3 grid((unsigned)((to - from + 3) / 4), (unsigned)m.BH);
  if (m.bf16) ring_fill_kernel<bf16><<<grid, 256, 0, st>>>(m, d, src, from, to);
  else ring_fill_kernel<float><<<grid, 256, 0, st>>>(m, d, src, from, to);
  return hipGetLastError();
}

hipError_t launch_decode(const Dims& m, const Dev& d, const void* q, const void* k, const void* v, const float* l,
                         int64_t t, int rows, void* out, hipStream_t st, const int64_t* seq) {
  const int64_t c = t / m.C;
  const int64_t lo = c * m.C - m.W > 0 ? c * m.C - m.W : 0;
  if (m.bf16)
    dec_kernel<bf16><<<m.BH, 64 * kDecWaves, 0, st>>>(m, d, reinterpret_cast<const bf16*>(q), reinterpret_cast<const bf16*>(k),
                                                     reinterpret_cast<const bf16*>(v), l, reinterpret_cast<bf16*>(out), t,
                                                     rows, lo, seq);
  else
    dec_kernel<float><<<m.BH, 64 * kDecWaves, 0, st>>>(m, d, reinterpret_cast<const float*>(q), reinterpret_cast<const float*>(k),
                                                      reinterpret_cast<const float*>(v), l, reinterpret_cast<float*>(out), t,
                                                      rows, lo, seq);
  return hipGetLastError();
}

hipError_t launch_snapshot_gather(const Dims& m, const Dev& d, int rows, int64_t ioff, int stride, void* key_out,
                                  void* val_out, float* rho_out, int* count_out, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  if (m.bf16)
    snapshot_gather_kernel<bf16><<<m.BH, 256, 0, st>>>(m, d, rows, ioff, stride, reinterpret_cast<f16*>(key_out),
                                                       reinterpret_cast<bf16*>(val_out), rho_out, count_out);
  else
    snapshot_gather_kernel<float><<<m.BH, 256, 0, st>>>(m, d, rows, ioff, stride, reinterpret_cast<float*>(key_out),
                                                         reinterpret_cast<float*>(val_out), rho_out, count_out);
  return hipGetLastError();
}

hipError_t launch_state_load(const Dims& m, const Dev& d, int rows, int64_t ioff, hipStream_t st) {
  if (m.bf16) state_load_kernel<bf16><<<m.BH, 256, 0, st>>>(m, d, rows, ioff);
  else state_load_kernel<float><<<m.BH, 256, 0, st>>>(m, d, rows, ioff);
  return hipGetLastError();
}

}  // namespace kvm
