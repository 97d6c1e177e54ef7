// gfx950 kernels of the Key-Value Means layer's backward pass.
//
// [KVM abstract]: the layer supports chunk-wise parallelizable training.  The
// gradient of a loss with respect to q, k, v and the gate logits is taken
// through the forward that kvm_prefill computed, with its discrete choices
// (the winner-take-all row of every merged token, the appended tokens, read
// back from the trace) held fixed:
//   bwd_q_kernel      per (sequence, query chunk): the joint softmax over
//                     [snapshot read form || window] recomputed (row maximum,
//                     then the row sum and D = sum_j P_j dP_j), then dq;
//   bwd_kv_kernel     per (sequence, query chunk): each wave owns key tiles and
//                     accumulates their dk and dv over the chunk's queries;
//                     the result is one partial per (chunk, key);
//   bwd_win_kernel    per token: the window keys' partials of the chunks that
//                     saw the key, RoPE transposed ([KVM summary, Core
//                     mechanisms 4]);
//   bwd_state_kernel  per state row: back through the read form of every
//                     snapshot (LayerNorm of K/n, the value at its radius;
//                     [KVM summary, Core mechanisms 2]) and the running sums of
//                     the chunk recurrence, last chunk first ([KVM lay summary,
//                     "smart merge"]: the sums only grow);
//   bwd_token_kernel  per absorbed token: merged tokens took g * (k, v) into
//                     their row, creators set it (and its radius |v|); the gate
//                     g = sigmoid(l) ([KVM summary, Core mechanisms 2]).
// Everything in fp32; contractions on v_mfma_f32_32x32x2f32.  Every gradient
// element is written by one thread in a fixed order: no float atomics, so the
// backward is bitwise repeatable.
//
// v_mfma_f32_32x32x2f32: lane l gives A[l%32][k_l] and B[k_l][l%32] with
// k_l = l/32 (or any bijection of the contraction index, used consistently by
// A and B); D lane l register r is D[row(r, l/32)][l%32], row(r, h) =
// 8(r/4) + 4h + r%4.  A score tile computed with keys as rows thus holds, in
// register r of lane l, exactly the A operand that a product contracting over
// those keys needs at step r (contraction index row(r, l/32)): dS and P feed
// the next products from registers, with no transpose through LDS.
#include <hip/hip_runtime.h>
#include <limits.h>
#include <math.h>
#include <type_traits>

#include "kvm_device.h"
#include "kvm_internal.h"

namespace kvm {
namespace {

__device__ __forceinline__ int mrow(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

constexpr int kPitch = 65;   // fp32 tile rows in LDS: 64 dims + 1 (rows land on distinct banks)

// Tile T of query chunk c's keys: state tiles (32 snapshot rows each) first,
// then window tiles (32 positions of [lo, hi) each).  Stages the keys (state:
// read-form key in columns 32..63, columns 0..31 zero; window: the rotated key
// kept by bwd_rot_kernel) and the values (state: read-form value; window: the
// input value) into LDS as fp32, zero past the end; 16-byte loads (4 dims per
// thread and row).
template <typename E>
__device__ __forceinline__ float4 load4(const E* p) {
  if constexpr (sizeof(E) == 4) {
    return *reinterpret_cast<const float4*>(p);
  } else {
    const uint2 x = *reinterpret_cast<const uint2*>(p);
    const E* e = reinterpret_cast<const E*>(&x);
    return make_float4(tof(e[0]), tof(e[1]), tof(e[2]), tof(e[3]));
  }
}

template <typename T, int PITCH = kPitch>
__device__ void bwd_stage(float* Kt, float* Vt, int Tile, int n_st, int S, const int* idxl, const Dims& m,
                          const Dev& d, const BwdIn& in, const Bwd& b, int s, int64_t lo, int64_t hi, int tid,
                          int nt) {
  using RT = typename Rd<T>::type;
  const RT* pk = reinterpret_cast<const RT*>(d.pkey) + (size_t)s * m.V_cap * 32;
  const T* pv = reinterpret_cast<const T*>(d.pval) + (size_t)s * m.V_cap * 64;
  const float* kr32 = b.kr32 + (size_t)s * in.N * 64;
  const T* vin = reinterpret_cast<const T*>(in.v) + (size_t)s * in.N * 64;
  for (int e = tid; e < 32 * 16; e += nt) {
    const int key = e >> 4, c4 = e & 15;
    float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), vv = kv;
    if (Tile < n_st) {
      const int r = Tile * 32 + key;
      if (r < S) {
        const int64_t ver = idxl[r];
        if (c4 >= 8) kv = load4(pk + ver * 32 + 4 * c4 - 32);
        vv = load4(pv + ver * 64 + 4 * c4);
      }
    } else {
      const int64_t pos = lo + (int64_t)(Tile - n_st) * 32 + key;
      if (pos < hi) {
        kv = *reinterpret_cast<const float4*>(kr32 + pos * 64 + 4 * c4);
        vv = load4(vin + pos * 64 + 4 * c4);
      }
    }
    float* kd = Kt + key * PITCH + 4 * c4;
    float* vd = Vt + key * PITCH + 4 * c4;
    kd[0] = kv.x; kd[1] = kv.y; kd[2] = kv.z; kd[3] = kv.w;
    vd[0] = vv.x; vd[1] = vv.y; vd[2] = vv.z; vd[3] = vv.w;
  }
}

// Rotated queries and keys of every position, fp32 (RoPE at the position,
// [KVM summary, Core mechanisms 4]): read by the tiles of several query
// chunks, so rotated once.  Eight threads per position, eight dims each (a
// thread on the rotary dims also reads its partner's eight, 16 dims away).
__device__ __forceinline__ void load8f(const float* p, float (&x)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p), c = *reinterpret_cast<const float4*>(p + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = c.x; x[5] = c.y; x[6] = c.z; x[7] = c.w;
}
__device__ __forceinline__ void load8f(const bf16* p, float (&x)[8]) {
  const bf16x8 a = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = (float)a[e];
}
template <typename T>
__global__ __launch_bounds__(256) void bwd_rot_kernel(Dims m, Dev d, BwdIn in, Bwd b) {
  const int s = blockIdx.y;
  const int64_t pos = (int64_t)blockIdx.x * 32 + (threadIdx.x >> 3);
  const int t8 = threadIdx.x & 7;
  if (pos >= in.N) return;
  const size_t r = ((size_t)s * in.N + pos) * 64;
  const int d0 = 8 * t8;
  float cs[8], sn[8];
  if (t8 < 4) {
    load8f(d.rope_cos + pos * 16 + (d0 & 15), cs);
    load8f(d.rope_sin + pos * 16 + (d0 & 15), sn);
  }
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    const T* src = reinterpret_cast<const T*>(which ? in.k : in.q) + r;
    float x[8];
    load8f(src + d0, x);
    if (t8 < 4) {   // pairs (j, j + 16) of the rotary dims: x' = x cos - x[j+16] sin, x[j+16]' = x[j+16] cos + x sin
      float y[8];
      load8f(src + (d0 ^ 16), y);
      const float sg = t8 < 2 ? -1.f : 1.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = fmaf(sg * y[e], sn[e], x[e] * cs[e]);
    }
    if (Is<T>::bf && which) {   // keys on the bf16 path: bf16 hi (dims 0..63) | lo (dims 0..63) per row
      bf16x8 hv, lv;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        hv[e] = (bf16)x[e];
        lv[e] = (bf16)(x[e] - (float)hv[e]);
      }
      bf16* dst = reinterpret_cast<bf16*>(b.kr32) + 2 * r + d0;
      *reinterpret_cast<bf16x8*>(dst) = hv;
      *reinterpret_cast<bf16x8*>(dst + 64) = lv;
    } else {
      float* dst = (which ? b.kr32 : b.qr32) + r + d0;
      *reinterpret_cast<float4*>(dst) = make_float4(x[0], x[1], x[2], x[3]);
      *reinterpret_cast<float4*>(dst + 4) = make_float4(x[4], x[5], x[6], x[7]);
    }
  }
}

// Tile validity of score element (key row kr of the tile, query at position qp).
__device__ __forceinline__ bool bwd_valid(int Tile, int n_st, int S, int64_t lo, int64_t hi, int key, int64_t qp,
                                          bool qvalid) {
  if (!qvalid) return false;
  if (Tile < n_st) return Tile * 32 + key < S;
  const int64_t pos = lo + (int64_t)(Tile - n_st) * 32 + key;
  return pos < hi && pos <= qp;
}

// ---------------------------------------------------------------------------
// dq.  One wave per 32 queries, lane l%32 = query; scores S^T = K . Q^T with the
// keys as rows.  Two sweeps over the key tiles: the row maximum, row sum and
// D = sum_j P_j dP_j (dP = dO . v_j) online, then dq += dS . K.
// ---------------------------------------------------------------------------
template <typename T, int NW>
__global__ __launch_bounds__(NW * 64) void bwd_q_kernel(Dims m, Dev d, BwdIn in, Bwd b) {
  constexpr int C = NW * 32;
  constexpr int NT = NW * 64;
  __shared__ float Kt[32 * kPitch], Vt[32 * kPitch];
  const int s = blockIdx.x % m.BH;
  const int c = blockIdx.x / m.BH;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, ql = lane & 31;
  const int64_t cpos = (int64_t)c * C;
  const int64_t qp = cpos + 32 * w + ql;
  const bool qvalid = qp < in.N;
  const int64_t qq = qvalid ? qp : in.N - 1;
  const float c2 = m.scale * kLog2e;
  // snapshot read by this chunk and its tiles
  const int64_t jj = c - m.W / C - 1;
  int S = 0;
  const int* idxl = d.idx + (size_t)s * m.idx_total;
  if (jj >= 0) {
    const int4 sc = d.sched[jj];
    S = sc.x + sc.y + sc.z;
    idxl += sc.w;
  }
  const int n_st = (S + 31) >> 5;
  const int64_t lo = cpos - m.W > 0 ? cpos - m.W : 0;
  const int64_t hi = cpos + C < in.N ? cpos + C : in.N;
  const int n_tiles = n_st + (int)((hi - lo + 31) >> 5);
  // query (rotated, scaled into log2 units) and dO, as B operands: step k takes dims 2k + h
  float qf[32], df[32];
  {
    const float* qr = b.qr32 + ((size_t)s * in.N + qq) * 64;
    const T* dor = reinterpret_cast<const T*>(in.dout) + ((size_t)s * in.N + qq) * 64;
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      const int dd = 2 * k + h;
      qf[k] = qr[dd] * c2;
      df[k] = qvalid ? tof(dor[dd]) : 0.f;
    }
  }
  auto scores = [&](int Tile) {
    f32x16 acc = {};
    const bool st = Tile < n_st;   // state keys live on dims 32..63 only
#pragma unroll
    for (int k = 0; k < 32; ++k)
      if (k >= 16 || !st) acc = mfma_f32(Kt[ql * kPitch + 2 * k + h], qf[k], acc);
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (!bwd_valid(Tile, n_st, S, lo, hi, mrow(r, h), qp, qvalid)) acc[r] = -kInf;
    return acc;
  };
  auto dscores = [&]() {
    f32x16 acc = {};
#pragma unroll
    for (int k = 0; k < 32; ++k) acc = mfma_f32(Vt[ql * kPitch + 2 * k + h], df[k], acc);
    return acc;
  };
  // sweep 1: the row maximum, row sum and D = sum_j P_j dP_j, online (the two
  // halves of a lane pair hold the same query and move their reference together)
  float mx = -kInf, ls = 0.f, ds = 0.f;
  for (int Tile = 0; Tile < n_tiles; ++Tile) {
    __syncthreads();
    bwd_stage<T>(Kt, Vt, Tile, n_st, S, idxl, m, d, in, b, s, lo, hi, tid, NT);
    __syncthreads();
    const f32x16 a = scores(Tile);
    const f32x16 dp = dscores();
    float mt = -kInf;
#pragma unroll
    for (int r = 0; r < 16; ++r) mt = fmaxf(mt, a[r]);
    mt = fmaxf(mt, partner_f(mt));
    const float mn = fmaxf(mx, mt);
    if (mn != -kInf) {
      const float al = mx == -kInf ? 0.f : exp2f(mx - mn);
      ls *= al;
      ds *= al;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = a[r] == -kInf ? 0.f : exp2f(a[r] - mn);
        ls += p;
        ds = fmaf(p, dp[r], ds);
      }
      mx = mn;
    }
  }
  ls += partner_f(ls);
  ds += partner_f(ds);
  const float lse = mx + log2f(ls);
  const float Dq = ds / ls;
  if (qvalid && h == 0) b.lse_d[(size_t)s * in.N + qp] = make_float2(lse, Dq);
  // sweep 2: dq += dS . K (contraction over the tile's keys in register order)
  f32x16 dq0 = {}, dq1 = {};
  for (int Tile = 0; Tile < n_tiles; ++Tile) {
    __syncthreads();
    bwd_stage<T>(Kt, Vt, Tile, n_st, S, idxl, m, d, in, b, s, lo, hi, tid, NT);
    __syncthreads();
    const f32x16 a = scores(Tile);
    const f32x16 dp = dscores();
    f32x16 dsc;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = a[r] == -kInf ? 0.f : exp2f(a[r] - lse);
      dsc[r] = p * (dp[r] - Dq);
    }
    if (Tile >= n_st) {
#pragma unroll
      for (int k = 0; k < 16; ++k) dq0 = mfma_f32(dsc[k], Kt[mrow(k, h) * kPitch + ql], dq0);
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) dq1 = mfma_f32(dsc[k], Kt[mrow(k, h) * kPitch + 32 + ql], dq1);
  }
  // dq rows are queries (register r: query row(r, h)), lane column = dim; RoPE transposed
  // on dims 0..31 (pair (j, j + 16): the partner is lane l ^ 16), natural-logit scale
  float* dqo = b.dq + (size_t)s * in.N * 64;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int64_t qpos = cpos + 32 * w + mrow(r, h);
    const float y = dq0[r];
    const float yp = __shfl_xor(y, 16);
    if (qpos < in.N) {
      const int jf = ql & 15;
      const float cs = d.rope_cos[qpos * 16 + jf], sn = d.rope_sin[qpos * 16 + jf];
      const float x = ql < 16 ? y * cs + yp * sn : y * cs - yp * sn;
      dqo[qpos * 64 + ql] = m.scale * x;
      dqo[qpos * 64 + 32 + ql] = m.scale * dq1[r];
    }
  }
}

// ---------------------------------------------------------------------------
// dk, dv partials of one query chunk.  The chunk's queries (rotated), dO, and
// their (lse, D) sit in LDS, in blocks of up to 128 queries; each wave owns key
// tiles (tile w, w + NW, ...) and contracts over the queries, so a key's
// partial is complete in one wave's registers.  S = Q . K^T with the queries as
// rows.
// ---------------------------------------------------------------------------
constexpr int kQB = 128;   // queries per LDS block

template <typename T, int NW>
__global__ __launch_bounds__(NW * 64) void bwd_kv_kernel(Dims m, Dev d, BwdIn in, Bwd b) {
  using RT = typename Rd<T>::type;
  constexpr int C = NW * 32;
  constexpr int QB = C < kQB ? C : kQB;
  __shared__ float Qs[QB * kPitch], Ds[QB * kPitch];
  __shared__ float2 LD[QB];
  const int s = blockIdx.x % m.BH;
  const int c = blockIdx.x / m.BH;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, kl = lane & 31;
  const int64_t cpos = (int64_t)c * C;
  const float c2 = m.scale * kLog2e;
  const int64_t jj = c - m.W / C - 1;
  int S = 0;
  int64_t ioff = 0;
  if (jj >= 0) {
    const int4 sc = d.sched[jj];
    S = sc.x + sc.y + sc.z;
    ioff = sc.w;
  }
  const int* idxl = d.idx + (size_t)s * m.idx_total + ioff;
  const int n_st = (S + 31) >> 5;
  const int64_t lo = cpos - m.W > 0 ? cpos - m.W : 0;
  const int64_t hi = cpos + C < in.N ? cpos + C : in.N;
  const int n_tiles = n_st + (int)((hi - lo + 31) >> 5);
  const RT* pk = reinterpret_cast<const RT*>(d.pkey) + (size_t)s * m.V_cap * 32;
  const T* pv = reinterpret_cast<const T*>(d.pval) + (size_t)s * m.V_cap * 64;
  const T* vin = reinterpret_cast<const T*>(in.v) + (size_t)s * in.N * 64;
  const T* doin = reinterpret_cast<const T*>(in.dout) + (size_t)s * in.N * 64;
  for (int q0 = 0; q0 < C; q0 += QB) {
    // the block's queries, rotated (unscaled), their dO and (lse, D); zero past the end
    __syncthreads();
    for (int e = tid; e < QB * 16; e += NW * 64) {
      const int qi = e >> 4, c4 = e & 15;
      const int64_t pos = cpos + q0 + qi;
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f), g = x;
      if (pos < in.N) {
        x = *reinterpret_cast<const float4*>(b.qr32 + ((size_t)s * in.N + pos) * 64 + 4 * c4);
        g = load4(doin + pos * 64 + 4 * c4);
      }
      float* qd = Qs + qi * kPitch + 4 * c4;
      float* gd = Ds + qi * kPitch + 4 * c4;
      qd[0] = x.x; qd[1] = x.y; qd[2] = x.z; qd[3] = x.w;
      gd[0] = g.x; gd[1] = g.y; gd[2] = g.z; gd[3] = g.w;
    }
    for (int qi = tid; qi < QB; qi += NW * 64) {
      const int64_t pos = cpos + q0 + qi;
      LD[qi] = pos < in.N ? b.lse_d[(size_t)s * in.N + pos] : make_float2(kInf, 0.f);
    }
    __syncthreads();
    for (int Tile = w; Tile < n_tiles; Tile += NW) {
      const bool st = Tile < n_st;
      // this wave's keys as B operands (step k: dims 2k + h) and their positions
      float kf[32], vf[32];
      int64_t kpos = 0;
      bool kvalid;
      if (st) {
        const int r = Tile * 32 + kl;
        kvalid = r < S;
        const int64_t ver = kvalid ? idxl[r] : 0;
#pragma unroll
        for (int k = 0; k < 32; ++k) {
          const int dd = 2 * k + h;
          kf[k] = kvalid && dd >= 32 ? tof(pk[ver * 32 + dd - 32]) : 0.f;
          vf[k] = kvalid ? tof(pv[ver * 64 + dd]) : 0.f;
        }
      } else {
        kpos = lo + (int64_t)(Tile - n_st) * 32 + kl;
        kvalid = kpos < hi;
        const int64_t pp = kvalid ? kpos : lo;
        const float* kr = b.kr32 + ((size_t)s * in.N + pp) * 64;
#pragma unroll
        for (int k = 0; k < 32; ++k) {
          const int dd = 2 * k + h;
          kf[k] = kvalid ? kr[dd] : 0.f;
          vf[k] = kvalid ? tof(vin[pp * 64 + dd]) : 0.f;
        }
      }
      f32x16 dk0 = {}, dk1 = {}, dv0 = {}, dv1 = {};
      for (int qs = 0; qs < QB; qs += 32) {
        f32x16 sc = {}, dp = {};
#pragma unroll
        for (int k = 0; k < 32; ++k)
          if (k >= 16 || !st) sc = mfma_f32(Qs[(qs + kl) * kPitch + 2 * k + h], kf[k], sc);
#pragma unroll
        for (int k = 0; k < 32; ++k) dp = mfma_f32(Ds[(qs + kl) * kPitch + 2 * k + h], vf[k], dp);
        f32x16 p, dsc;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qi = qs + mrow(r, h);
          const int64_t qpos = cpos + q0 + qi;
          const float2 ld = LD[qi];
          const bool ok = kvalid && qpos < in.N && (st || kpos <= qpos);
          const float pr = ok ? exp2f(sc[r] * c2 - ld.x) : 0.f;
          p[r] = pr;
          dsc[r] = pr * (dp[r] - ld.y);
        }
        // dk[key][d] += dS^T . Q, dv[key][e] += P^T . dO: contraction over the sub-block's
        // queries in register order (query row(k, h) at step k)
        if (!st) {
#pragma unroll
          for (int k = 0; k < 16; ++k) dk0 = mfma_f32(dsc[k], Qs[(qs + mrow(k, h)) * kPitch + kl], dk0);
        }
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const int qrow = (qs + mrow(k, h)) * kPitch;
          dk1 = mfma_f32(dsc[k], Qs[qrow + 32 + kl], dk1);
          dv0 = mfma_f32(p[k], Ds[qrow + kl], dv0);
          dv1 = mfma_f32(p[k], Ds[qrow + 32 + kl], dv1);
        }
      }
      // rows of the results are keys (register r: key row(r, h)), lane column = dim.  The
      // first query block writes the partial, later blocks add to it (same wave, in order).
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = mrow(r, h);
        float* dst;
        if (st) {
          const int row = Tile * 32 + key;
          if (row >= S) continue;
          dst = b.part_state + ((size_t)s * m.idx_total + ioff + row) * 96;
          const float a0 = m.scale * dk1[r], a1 = dv0[r], a2 = dv1[r];
          if (q0 == 0) {
            dst[kl] = a0;
            dst[32 + kl] = a1;
            dst[64 + kl] = a2;
          } else {
            dst[kl] += a0;
            dst[32 + kl] += a1;
            dst[64 + kl] += a2;
          }
        } else {
          const int64_t pos = lo + (int64_t)(Tile - n_st) * 32 + key;
          if (pos >= hi) continue;
          const int64_t off = pos - (cpos - m.W);   // in [0, W + C)
          dst = b.part_win + (((size_t)s * b.nq + c) * m.R + off) * 128;
          const float a0 = m.scale * dk0[r], a1 = m.scale * dk1[r], a2 = dv0[r], a3 = dv1[r];
          if (q0 == 0) {
            dst[kl] = a0;
            dst[32 + kl] = a1;
            dst[64 + kl] = a2;
            dst[96 + kl] = a3;
          } else {
            dst[kl] += a0;
            dst[32 + kl] += a1;
            dst[64 + kl] += a2;
            dst[96 + kl] += a3;
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 path: the same two kernels with the products on 16-bit operands
// (v_mfma_f32_32x32x16_{bf16,f16}, fp32 accumulation), as in the forward:
// window scores from bf16 rotated keys and bf16 queries, state scores from the
// fp16 read-form keys and fp16 queries (an exact power-of-two pre-scale keeps
// the query in fp16 range), dP from the bf16 values and dO (exact), and the
// second-stage products (dq = dS . K, dk = dS^T . Q, dv = P^T . dO) with the
// fp32 factors (P, dS, the rotated keys and queries) as hi + lo bf16 pairs, so
// that they keep ~2^-16 of their precision.  Tiles sit in LDS as 16-bit rows.
// MFMA step kk contracts 16 keys (or queries); lane half h supplies the eight
// that its score registers 8 kk .. 8 kk + 7 hold (rows mrow(8 kk + i, h)), and
// the other operand is read for the same eight rows, so the score registers
// feed the next product directly, as in the fp32 kernels.
// ---------------------------------------------------------------------------
constexpr int kRP = 72;   // row-major 16-bit tile rows (halves): 144 B, 16 lanes' 16-byte reads on distinct banks
constexpr int kTP = 40;   // 16-bit rows of 32 halves (+ 8): 80 B, likewise
constexpr int kBwdIdxCap = 4096;   // snapshot rows whose version ids the bf16 kernels keep in LDS

// x = hi + lo to ~2^-16 relative (bf16 hi, bf16 remainder)
__device__ __forceinline__ void bf8_split(const float (&x)[8], bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    hi[i] = (bf16)x[i];
    lo[i] = (bf16)(x[i] - (float)hi[i]);
  }
}
// 16-byte unit swizzle of a 128-byte tile row read by ds_read_b64_tr_b16: the
// 16 lanes of one LDS cycle read four consecutive rows two units each, so rows
// 0..3 (and 4..7) take disjoint unit pairs
__device__ __forceinline__ int tr_swz(int r) { return ((r & 3) << 1) | ((r >> 2) & 1); }
__device__ __forceinline__ bf16x4 tr_read(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)(p));
}
// power-of-two pre-scale exponent keeping values of magnitude < 2^14 * 2^qsh in fp16
__device__ __forceinline__ int f16_shift(float amax) {
  if (!(amax >= 16384.f)) return 0;
  int ex;
  frexpf(amax, &ex);
  return ex - 14;
}

template <int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2))) void bwd_q_mx_kernel(Dims m, Dev d, BwdIn in, Bwd b) {
  constexpr int C = NW * 32;
  constexpr int NT = NW * 64;
  // tile in LDS, 16-bit: keys row-major (fp16 for a state tile, bf16 for a
  // window tile; rows of kRP halves), values row-major (bf16), and the keys
  // again as hi + lo bf16 pairs in 128-byte rows with their 16-byte units
  // swizzled (tr_swz), read transposed by ds_read_b64_tr_b16 as the B operand
  // of dq = dS . K (keys along the contraction)
  __shared__ __attribute__((aligned(16))) uint16_t Kr[32 * kRP];
  __shared__ __attribute__((aligned(16))) uint16_t Vr[32 * kRP];
  __shared__ __attribute__((aligned(16))) uint8_t Kh[32 * 128];
  __shared__ __attribute__((aligned(16))) uint8_t Kl[32 * 128];
  __shared__ int sIdx[kBwdIdxCap];   // the snapshot's version ids (one load round trip per tile, not two)
  const int s = blockIdx.x % m.BH;
  const int c = blockIdx.x / m.BH;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, ql = lane & 31;
  const int64_t cpos = (int64_t)c * C;
  const int64_t qp = cpos + 32 * w + ql;
  const bool qvalid = qp < in.N;
  const int64_t qq = qvalid ? qp : in.N - 1;
  const float c2 = m.scale * kLog2e;
  const int64_t jj = c - m.W / C - 1;
  int S = 0;
  const int* idxl = d.idx + (size_t)s * m.idx_total;
  if (jj >= 0) {
    const int4 sc = d.sched[jj];
    S = sc.x + sc.y + sc.z;
    idxl += sc.w;
  }
  const int n_st = (S + 31) >> 5;
  for (int i = tid; i < S && i < kBwdIdxCap; i += NT) sIdx[i] = idxl[i];
  __syncthreads();
  const int64_t lo = cpos - m.W > 0 ? cpos - m.W : 0;
  const int64_t hi = cpos + C < in.N ? cpos + C : in.N;
  const int n_tiles = n_st + (int)((hi - lo + 31) >> 5);
  // B operands: the query (rotated, scaled into log2 units; bf16 for the window,
  // fp16 on the state's dims 32..63) and dO, step kk taking dims 16 kk + 8 h + e
  bf16x8 qb[4], db[4];
  f16x8 qh[2];
  int qsh;
  {
    const float* qr = b.qr32 + ((size_t)s * in.N + qq) * 64;
    const bf16* dor = reinterpret_cast<const bf16*>(in.dout) + ((size_t)s * in.N + qq) * 64;
    float amax = 0.f;
    float xs[4][8];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const float4 a = *reinterpret_cast<const float4*>(qr + 16 * kk + 8 * h);
      const float4 b2 = *reinterpret_cast<const float4*>(qr + 16 * kk + 8 * h + 4);
      const float y[8] = {a.x, a.y, a.z, a.w, b2.x, b2.y, b2.z, b2.w};
      const bf16x8 dv = *reinterpret_cast<const bf16x8*>(dor + 16 * kk + 8 * h);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = y[e] * c2;
        xs[kk][e] = x;
        qb[kk][e] = (bf16)x;
        if (kk >= 2) amax = fmaxf(amax, fabsf(x));
      }
      db[kk] = qvalid ? dv : bf16x8{};
    }
    amax = fmaxf(amax, partner_f(amax));
    qsh = f16_shift(amax);
    const float sc = ldexpf(1.f, -qsh);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) qh[kk][e] = (f16)(xs[2 + kk][e] * sc);
  }
  const float qscale = ldexpf(1.f, qsh);
  const bool wave_qsh = __ballot(qsh != 0) != 0ull;
  // Tile staging through registers: the next tile's loads are issued right
  // after the barrier that publishes this one, so they travel while this tile
  // is computed.  Each thread holds IT pieces of four dims of keys (raw, 16
  // bytes either way) and of values (bf16), converted only when stored, so
  // that no wait follows the loads.
  constexpr int IT = 32 * 16 / NT;
  uint4 rk[IT];   // window: four dims as bf16 hi (x, y) and lo (z, w); state: eight fp16 dims holding the four
  uint2 rv[IT];
  const f16* pk = reinterpret_cast<const f16*>(d.pkey) + (size_t)s * m.V_cap * 32;
  const bf16* pv = reinterpret_cast<const bf16*>(d.pval) + (size_t)s * m.V_cap * 64;
  const bf16* krh = reinterpret_cast<const bf16*>(b.kr32) + (size_t)s * in.N * 128;   // rows: hi 64 | lo 64
  const bf16* vin = reinterpret_cast<const bf16*>(in.v) + (size_t)s * in.N * 64;
  const bool idx_lds = S <= kBwdIdxCap;   // (uniform) version ids from LDS
  // (loads are unconditional, at clamped in-range addresses, and a piece's
  // validity is kept beside it and applied when it is stored: a load under a
  // lane-dependent branch would be waited for where the branch joins)
  uint32_t rok = 0u;   // bit it: piece it's key and value are real (else zero)
  auto load_tile = [&](int Tile, auto from_lds) __attribute__((always_inline)) {
    rok = 0u;
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int e = tid + it * NT, key = e >> 4, c4 = e & 15;
      const bf16* va;
      if (Tile < n_st) {
        const int r = Tile * 32 + key;
        const int rc = r < S ? r : S - 1;
        int64_t ver;
        if constexpr (decltype(from_lds)::value) ver = sIdx[rc];
        else ver = idxl[rc];
        // (a 16-byte read inside the row: dims 4 (c4 & 7) .. + 7, or 24 .. 31 for the last piece)
        const int k0 = (c4 & 7) == 7 ? 24 : 4 * (c4 & 7);
        rk[it] = *reinterpret_cast<const uint4*>(pk + ver * 32 + k0);
        va = pv + ver * 64 + 4 * c4;
        rok |= (r < S ? 1u : 0u) << it;
      } else {
        const int64_t pos = lo + (int64_t)(Tile - n_st) * 32 + key;
        const int64_t pc = pos < hi ? pos : hi - 1;
        const uint2 kh2 = *reinterpret_cast<const uint2*>(krh + pc * 128 + 4 * c4);
        const uint2 kl2 = *reinterpret_cast<const uint2*>(krh + pc * 128 + 64 + 4 * c4);
        rk[it] = make_uint4(kh2.x, kh2.y, kl2.x, kl2.y);
        va = vin + pc * 64 + 4 * c4;
        rok |= (pos < hi ? 1u : 0u) << it;
      }
      rv[it] = *reinterpret_cast<const uint2*>(va);
    }
  };
  auto prefetch = [&](int Tile) __attribute__((always_inline)) {
    if (idx_lds) load_tile(Tile, std::true_type{});
    else load_tile(Tile, std::false_type{});
  };
  auto store_tile = [&](int Tile) __attribute__((always_inline)) {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int e = tid + it * NT, key = e >> 4, c4 = e & 15;
      const bool ok = (rok >> it) & 1u;
      uint2 hb, lb;   // the piece's keys as bf16 hi and lo bits
      if (Tile < n_st) {   // fp16 bits as they are (zero on dims 0..31), split into hi + lo
        const bool kok = ok && c4 >= 8;
        const uint2 kr2 = (c4 & 7) == 7 ? make_uint2(rk[it].z, rk[it].w) : make_uint2(rk[it].x, rk[it].y);
        const uint2 k2 = kok ? kr2 : make_uint2(0u, 0u);
        *reinterpret_cast<uint2*>(Kr + key * kRP + 4 * c4) = k2;
        const f16x4 k4 = __builtin_bit_cast(f16x4, k2);
        bf16x4 h4, l4;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float kx = (float)k4[t];
          h4[t] = (bf16)kx;
          l4[t] = (bf16)(kx - (float)h4[t]);
        }
        hb = __builtin_bit_cast(uint2, h4);
        lb = __builtin_bit_cast(uint2, l4);
      } else {
        hb = ok ? make_uint2(rk[it].x, rk[it].y) : make_uint2(0u, 0u);
        lb = ok ? make_uint2(rk[it].z, rk[it].w) : make_uint2(0u, 0u);
        *reinterpret_cast<uint2*>(Kr + key * kRP + 4 * c4) = hb;
      }
      *reinterpret_cast<uint2*>(Vr + key * kRP + 4 * c4) = ok ? rv[it] : make_uint2(0u, 0u);
      const int o = key * 128 + 16 * ((c4 >> 1) ^ tr_swz(key)) + 8 * (c4 & 1);
      *reinterpret_cast<uint2*>(Kh + o) = hb;
      *reinterpret_cast<uint2*>(Kl + o) = lb;
    }
  };
  // B operand of dq at step kk: lane group g = lane / 16 reads keys
  // 16 kk + 4 h + (lane % 16) / 4 (and + 8) at dims 32 half + 16 (g % 2) + 4 (lane % 4);
  // the transposed read hands lane l dim 32 half + l % 32 of those keys
  int toff[2];
  {
    const int g = lane >> 4, pl = lane & 15;
    const int kq = 4 * h + (pl >> 2);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int d0 = 32 * half + 16 * (g & 1) + 4 * (pl & 3);
      toff[half] = kq * 128 + 16 * ((d0 >> 3) ^ tr_swz(kq)) + 8 * ((d0 >> 2) & 1);
    }
  }
  auto kfrag = [&](const uint8_t* T, int kk, int half) __attribute__((always_inline)) {
    const uint8_t* base = T + 16 * kk * 128 + toff[half];
    const bf16x4 a = tr_read(base), c = tr_read(base + 8 * 128);
    return bf16x8{a[0], a[1], a[2], a[3], c[0], c[1], c[2], c[3]};
  };
  // Masks are needed only on a tile that holds rows past the state's end, keys
  // past the window's end or after one of the wave's queries, or when some of
  // the wave's queries are past the end (all wave-uniform)
  const bool wave_q_all = __ballot(!qvalid) == 0ull;
  const int64_t wq0 = cpos + 32 * w;
  auto tile_masked = [&](int Tile) {
    if (!wave_q_all) return true;
    if (Tile < n_st) return Tile * 32 + 32 > S;
    const int64_t last = lo + (int64_t)(Tile - n_st) * 32 + 31;
    return last >= hi || last > wq0;
  };
  auto scores = [&](int Tile) {
    f32x16 acc = {};
    const uint16_t* kr = Kr + ql * kRP + 8 * h;
    if (Tile < n_st) {   // state keys live on dims 32..63 only
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        acc = mfma_f16(*reinterpret_cast<const f16x8*>(kr + 32 + 16 * kk), qh[kk], acc);
      if (wave_qsh) {
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] *= qscale;
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) acc = mfma_bf16(*reinterpret_cast<const bf16x8*>(kr + 16 * kk), qb[kk], acc);
    }
    if (tile_masked(Tile)) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (!bwd_valid(Tile, n_st, S, lo, hi, mrow(r, h), qp, qvalid)) acc[r] = -kInf;
    }
    return acc;
  };
  auto dscores = [&]() {
    f32x16 acc = {};
    const uint16_t* vr = Vr + ql * kRP + 8 * h;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) acc = mfma_bf16(*reinterpret_cast<const bf16x8*>(vr + 16 * kk), db[kk], acc);
    return acc;
  };
  // One sweep over the key tiles, online.  With weights e_j = 2^(s_j - m)
  // against a per-query reference m (moved only when a tile's maximum passes
  // it by more than 8, i.e. weights stay below 2^8; the sums are rescaled
  // then), it gathers l = sum e_j, t = sum e_j dP_j, A = sum e_j dP_j k_j and
  // B = sum e_j k_j.  Then P_j = e_j / l, D = t / l, and
  // dq = sum_j P_j (dP_j - D) k_j = (A - D B) / l.  A common offset of the
  // keys cancels in A - D B (as it does in sum_j dS_j k_j, whose dS sum to
  // 0), so the weights and the keys go in as hi + lo bf16 pairs (three
  // products each, to ~2^-16), not rounded once to bf16.
  float mref = -kInf, ls = 0.f, ds = 0.f;
  f32x16 A0 = {}, A1 = {}, B0 = {}, B1 = {};
  if (n_tiles > 0) prefetch(0);
  for (int Tile = 0; Tile < n_tiles; ++Tile) {
    __syncthreads();
    store_tile(Tile);
    __syncthreads();
    if (Tile + 1 < n_tiles) prefetch(Tile + 1);
    const f32x16 a = scores(Tile);
    const f32x16 dp = dscores();
    float mt = -kInf;
#pragma unroll
    for (int r = 0; r < 16; ++r) mt = fmaxf(mt, a[r]);
    mt = fmaxf(mt, partner_f(mt));
    const bool up = mt > mref + 8.f;   // (the first finite maximum sets the reference)
    if (__ballot(up) != 0ull) {
      const float mn = up ? mt : mref;
      const float al = mref == -kInf ? 0.f : exp2_fast(mref - mn);
      ls *= al;
      ds *= al;
      // register r holds query mrow(r, h), whose factor sits in lane mrow(r, h)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float ar = __shfl(al, mrow(r, h));
        A0[r] *= ar;
        A1[r] *= ar;
        B0[r] *= ar;
        B1[r] *= ar;
      }
      mref = mn;
    }
    const float mb = mref == -kInf ? 0.f : mref;   // (no valid score yet: the weights are 0)
    f32x16 e, wgt;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      e[r] = exp2_fast(a[r] - mb);   // (0 for a masked score)
      ls += e[r];
      ds = fmaf(e[r], dp[r], ds);
      wgt[r] = e[r] * dp[r];
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      float xe[8], xw[8];
      bf16x8 eh, el, wh, wl;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        xe[i] = e[8 * kk + i];
        xw[i] = wgt[8 * kk + i];
      }
      bf8_split(xe, eh, el);
      bf8_split(xw, wh, wl);
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        if (half == 0 && Tile < n_st) continue;   // state keys are zero on dims 0..31
        const bf16x8 bh = kfrag(Kh, kk, half), bl = kfrag(Kl, kk, half);
        f32x16& Aa = half ? A1 : A0;
        f32x16& Bb = half ? B1 : B0;
        Aa = mfma_bf16(wh, bh, Aa);
        Aa = mfma_bf16(wh, bl, Aa);
        Aa = mfma_bf16(wl, bh, Aa);
        Bb = mfma_bf16(eh, bh, Bb);
        Bb = mfma_bf16(eh, bl, Bb);
        Bb = mfma_bf16(el, bh, Bb);
      }
    }
  }
  ls += partner_f(ls);
  ds += partner_f(ds);
  const float lse = mref + log2f(ls);
  const float Dq = ds / ls;
  if (qvalid && h == 0) b.lse_d[(size_t)s * in.N + qp] = make_float2(lse, Dq);
  // (a query past the end has no valid score and no stored gradient)
  const float il = qvalid ? 1.f / ls : 0.f, Du = qvalid ? Dq : 0.f;
  f32x16 dq0, dq1;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const float dr = __shfl(Du, mrow(r, h)), ir = __shfl(il, mrow(r, h));
    dq0[r] = fmaf(-dr, B0[r], A0[r]) * ir;
    dq1[r] = fmaf(-dr, B1[r], A1[r]) * ir;
  }
  // dq rows are queries (register r: query row(r, h)), lane column = dim; RoPE transposed
  float* dqo = b.dq + (size_t)s * in.N * 64;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int64_t qpos = cpos + 32 * w + mrow(r, h);
    const float y = dq0[r];
    const float yp = __shfl_xor(y, 16);
    if (qpos < in.N) {
      const int jf = ql & 15;
      const float cs = d.rope_cos[qpos * 16 + jf], sn = d.rope_sin[qpos * 16 + jf];
      const float x = ql < 16 ? y * cs + yp * sn : y * cs - yp * sn;
      dqo[qpos * 64 + ql] = m.scale * x;
      dqo[qpos * 64 + 32 + ql] = m.scale * dq1[r];
    }
  }
}

// NV waves share the block's key tiles: the snapshot's state rows and (WIN)
// the window keys, whose partials go to part_win; without WIN the window keys
// are left to bwd_kvw_mx_kernel, and the LDS (~75 KB) lets two workgroups
// share a CU, so that one's staging overlaps the other's products.
template <int NW, int NV, bool WIN = true>
__global__ __launch_bounds__(NV * 64) __attribute__((amdgpu_waves_per_eu(2))) void bwd_kv_mx_kernel(
    Dims m, Dev d, BwdIn in, Bwd b) {
  constexpr int C = NW * 32;
  // query blocks of QB in LDS, 16-bit: queries row-major (bf16 for the window
  // scores, WIN only; fp16 pre-scaled on dims 32..63 for the state scores) as
  // the score products' A operands, and the queries as hi + lo planes and dO
  // in 128-byte rows with swizzled 16-byte units: read directly (dO, the A
  // operand of dP) and transposed (ds_read_b64_tr_b16) as the B operands of
  // dk and dv
  constexpr int QB = C < kQB ? C : kQB;
  __shared__ __attribute__((aligned(16))) uint16_t Qb[WIN ? QB * kRP : 8];
  __shared__ __attribute__((aligned(16))) uint16_t Qh[QB * kTP];
  __shared__ __attribute__((aligned(16))) uint8_t Th[QB * 128];
  __shared__ __attribute__((aligned(16))) uint8_t Tl[QB * 128];
  __shared__ __attribute__((aligned(16))) uint8_t Td[QB * 128];
  __shared__ float2 LD[QB];
  __shared__ unsigned qmax_bits;
  __shared__ int sIdx[kBwdIdxCap];   // the snapshot's version ids
  const int s = blockIdx.x % m.BH;
  const int c = blockIdx.x / m.BH;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, kl = lane & 31;
  const int64_t cpos = (int64_t)c * C;
  const float c2 = m.scale * kLog2e;
  const int64_t jj = c - m.W / C - 1;
  int S = 0;
  int64_t ioff = 0;
  if (jj >= 0) {
    const int4 sc = d.sched[jj];
    S = sc.x + sc.y + sc.z;
    ioff = sc.w;
  }
  const int* idxl = d.idx + (size_t)s * m.idx_total + ioff;
  const int n_st = (S + 31) >> 5;
  for (int i = tid; i < S && i < kBwdIdxCap; i += NV * 64) sIdx[i] = idxl[i];
  const int64_t lo = cpos - m.W > 0 ? cpos - m.W : 0;
  const int64_t hi = cpos + C < in.N ? cpos + C : in.N;
  const int n_tiles = n_st + (WIN ? (int)((hi - lo + 31) >> 5) : 0);
  if (!WIN && n_st == 0) return;   // (no state rows before this chunk: nothing to do)
  const f16* pk = reinterpret_cast<const f16*>(d.pkey) + (size_t)s * m.V_cap * 32;
  const bf16* pv = reinterpret_cast<const bf16*>(d.pval) + (size_t)s * m.V_cap * 64;
  const bf16* vin = reinterpret_cast<const bf16*>(in.v) + (size_t)s * in.N * 64;
  const bf16* doin = reinterpret_cast<const bf16*>(in.dout) + (size_t)s * in.N * 64;
  for (int q0 = 0; q0 < C; q0 += QB) {
    // the block's queries, rotated (unscaled), their dO and (lse, D); zero past the end
    __syncthreads();
    if (tid == 0) qmax_bits = 0u;
    __syncthreads();
    float amax = 0.f;
    for (int e = tid; e < QB * 16; e += NV * 64) {
      const int qi = e >> 4, c4 = e & 15;
      const int64_t pos = cpos + q0 + qi;
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
      uint2 g = make_uint2(0u, 0u);
      if (pos < in.N) {
        x = *reinterpret_cast<const float4*>(b.qr32 + ((size_t)s * in.N + pos) * 64 + 4 * c4);
        g = *reinterpret_cast<const uint2*>(doin + pos * 64 + 4 * c4);
      }
      if (c4 >= 8) amax = fmaxf(amax, fmaxf(fmaxf(fabsf(x.x), fabsf(x.y)), fmaxf(fabsf(x.z), fabsf(x.w))));
      const bf16x4 h4{(bf16)x.x, (bf16)x.y, (bf16)x.z, (bf16)x.w};
      const bf16x4 l4{(bf16)(x.x - (float)h4[0]), (bf16)(x.y - (float)h4[1]), (bf16)(x.z - (float)h4[2]),
                      (bf16)(x.w - (float)h4[3])};
      if constexpr (WIN) *reinterpret_cast<bf16x4*>(Qb + qi * kRP + 4 * c4) = h4;
      const int o = qi * 128 + 16 * ((c4 >> 1) ^ tr_swz(qi)) + 8 * (c4 & 1);
      *reinterpret_cast<bf16x4*>(Th + o) = h4;
      *reinterpret_cast<bf16x4*>(Tl + o) = l4;
      *reinterpret_cast<uint2*>(Td + o) = g;
    }
    atomicMax(&qmax_bits, __float_as_uint(amax));   // non-negative floats order as their bits
    for (int qi = tid; qi < QB; qi += NV * 64) {
      const int64_t pos = cpos + q0 + qi;
      LD[qi] = pos < in.N ? b.lse_d[(size_t)s * in.N + pos] : make_float2(kInf, 0.f);
    }
    __syncthreads();
    // state scores take the queries in fp16, pre-scaled by 2^-qsh (the same for
    // the block; dims 32..63 read again, now that the block maximum is known)
    const int qsh = f16_shift(__uint_as_float(qmax_bits));
    const float qdown = ldexpf(1.f, -qsh), qup = ldexpf(1.f, qsh);
    for (int e = tid; e < QB * 8; e += NV * 64) {
      const int qi = e >> 3, c4 = e & 7;
      const int64_t pos = cpos + q0 + qi;
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
      if (pos < in.N) x = *reinterpret_cast<const float4*>(b.qr32 + ((size_t)s * in.N + pos) * 64 + 32 + 4 * c4);
      *reinterpret_cast<f16x4*>(Qh + qi * kTP + 4 * c4) =
          f16x4{(f16)(x.x * qdown), (f16)(x.y * qdown), (f16)(x.z * qdown), (f16)(x.w * qdown)};
    }
    __syncthreads();
    // This wave's keys and values as B operands (step kk: dims 16 kk + 8 h + e;
    // 16-byte loads of eight consecutive dims).  A key past the end reads a
    // valid row: its scores are masked, so its weights are 0, and its
    // gradient is not stored.  The next tile's operands are loaded into the
    // same registers as soon as the last sub-block's score products have read
    // them, before this tile's stores, so that the wait for them at the next
    // tile does not wait for the stores too.
    bf16x8 kb[4], vb[4];
    f16x8 kh[2];
    // B operand of dk, dv at step kk: lane group g = lane / 16 reads queries
    // qs + 16 kk + 4 h + (lane % 16) / 4 (and + 8) at dims 32 half + 16 (g % 2) +
    // 4 (lane % 4); the transposed read hands lane l dim 32 half + l % 32
    auto qfrag = [&](const uint8_t* T, int qs, int kk, int half) __attribute__((always_inline)) {
      const int g = lane >> 4, pl = lane & 15;
      const int kq = 4 * h + (pl >> 2);
      const int d0 = 32 * half + 16 * (g & 1) + 4 * (pl & 3);
      const uint8_t* base = T + (qs + 16 * kk + kq) * 128 + 16 * ((d0 >> 3) ^ tr_swz(kq)) + 8 * ((d0 >> 2) & 1);
      const bf16x4 a = tr_read(base), c = tr_read(base + 8 * 128);
      return bf16x8{a[0], a[1], a[2], a[3], c[0], c[1], c[2], c[3]};
    };
    const bool idx_lds = S <= kBwdIdxCap;   // (uniform) version ids from LDS
    auto load_ops = [&](int Tile) __attribute__((always_inline)) {
      if (Tile < n_st) {
        const int r = Tile * 32 + kl;
        const int rr = r < S ? r : S - 1;
        const int64_t ver = idx_lds ? sIdx[rr] : idxl[rr];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) vb[kk] = *reinterpret_cast<const bf16x8*>(pv + ver * 64 + 16 * kk + 8 * h);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) kh[kk] = *reinterpret_cast<const f16x8*>(pk + ver * 32 + 16 * kk + 8 * h);
      } else {
        const int64_t kq = lo + (int64_t)(Tile - n_st) * 32 + kl;
        const int64_t pp = kq < hi ? kq : hi - 1;
        const bf16* kr = reinterpret_cast<const bf16*>(b.kr32) + ((size_t)s * in.N + pp) * 128;   // the hi plane
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          kb[kk] = *reinterpret_cast<const bf16x8*>(kr + 16 * kk + 8 * h);
          vb[kk] = *reinterpret_cast<const bf16x8*>(vin + pp * 64 + 16 * kk + 8 * h);
        }
      }
    };
    if (w < n_tiles) load_ops(w);
    for (int Tile = w; Tile < n_tiles; Tile += NV) {
      const bool st = !WIN || Tile < n_st;   // (without WIN every tile is a state tile)
      const int64_t kpos = lo + (int64_t)(Tile - n_st) * 32 + kl;    // (window tiles)
      const bool kvalid = st ? Tile * 32 + kl < S : kpos < hi;
      const int64_t klast = lo + (int64_t)(Tile - n_st) * 32 + 31;   // (window tiles) the tile's last key
      f32x16 dk0 = {}, dk1 = {}, dv0 = {}, dv1 = {};
      for (int qs = 0; qs < QB; qs += 32) {
        // S = Q . K^T and dP = dO . V^T, queries as rows (A operand rows qs + kl)
        const uint16_t* qrow = Qb + (qs + kl) * kRP + 8 * h;
        const uint16_t* hrow = Qh + (qs + kl) * kTP + 8 * h;
        const uint8_t* drow = Td + (qs + kl) * 128;   // (16-byte unit 2 kk + h, swizzled)
        f32x16 sc = {}, dp = {};
        if (st) {
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) sc = mfma_f16(*reinterpret_cast<const f16x8*>(hrow + 16 * kk), kh[kk], sc);
          if (qsh != 0) {
#pragma unroll
            for (int r = 0; r < 16; ++r) sc[r] *= qup;
          }
        } else {
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) sc = mfma_bf16(*reinterpret_cast<const bf16x8*>(qrow + 16 * kk), kb[kk], sc);
        }
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          dp = mfma_bf16(*reinterpret_cast<const bf16x8*>(drow + 16 * ((2 * kk + h) ^ tr_swz(kl))), vb[kk], dp);
        if (qs + 32 == QB && Tile + NV < n_tiles) load_ops(Tile + NV);
        // (a query past the end has lse = +inf, so its weights come out 0; the
        // mask is needed only on a ragged tile or one with keys after some of
        // the sub-block's queries: wave-uniform)
        f32x16 p, dsc;
        const bool need = st ? Tile * 32 + 32 > S : klast >= hi || klast > cpos + q0 + qs;
        if (need) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int qi = qs + mrow(r, h);
            const int64_t qpos = cpos + q0 + qi;
            const float2 ld = LD[qi];
            const bool ok = kvalid && (st || kpos <= qpos);
            const float pr = ok ? exp2_fast(sc[r] * c2 - ld.x) : 0.f;
            p[r] = pr;
            dsc[r] = pr * (dp[r] - ld.y);
          }
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float2 ld = LD[qs + mrow(r, h)];
            const float pr = exp2_fast(sc[r] * c2 - ld.x);
            p[r] = pr;
            dsc[r] = pr * (dp[r] - ld.y);
          }
        }
        // dk[key][d] += dS^T . Q (dS and Q as hi + lo pairs, three products) and
        // dv[key][e] += P^T . dO (P as a hi + lo pair, dO exact in bf16) over
        // the sub-block's queries
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          float xa[8];
          bf16x8 dh, dl, ph, pl, bh, bl;
#pragma unroll
          for (int i = 0; i < 8; ++i) xa[i] = dsc[8 * kk + i];
          bf8_split(xa, dh, dl);
#pragma unroll
          for (int i = 0; i < 8; ++i) xa[i] = p[8 * kk + i];
          bf8_split(xa, ph, pl);
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            f32x16& dk = half ? dk1 : dk0;
            f32x16& dv = half ? dv1 : dv0;
            if (half == 1 || !st) {   // state keys have no gradient on dims 0..31
              bh = qfrag(Th, qs, kk, half);
              bl = qfrag(Tl, qs, kk, half);
              dk = mfma_bf16(dh, bh, dk);
              dk = mfma_bf16(dh, bl, dk);
              dk = mfma_bf16(dl, bh, dk);
            }
            const bf16x8 od = qfrag(Td, qs, kk, half);
            dv = mfma_bf16(ph, od, dv);
            dv = mfma_bf16(pl, od, dv);
          }
        }
      }
      // rows of the results are keys (register r: key row(r, h)), lane column = dim
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = mrow(r, h);
        float* dst;
        if (st) {
          const int row = Tile * 32 + key;
          if (row >= S) continue;
          dst = b.part_state + ((size_t)s * m.idx_total + ioff + row) * 96;
          const float a0 = m.scale * dk1[r], a1 = dv0[r], a2 = dv1[r];
          if (q0 == 0) {
            dst[kl] = a0;
            dst[32 + kl] = a1;
            dst[64 + kl] = a2;
          } else {
            dst[kl] += a0;
            dst[32 + kl] += a1;
            dst[64 + kl] += a2;
          }
        } else {
          const int64_t pos = lo + (int64_t)(Tile - n_st) * 32 + key;
          if (pos >= hi) continue;
          const int64_t off = pos - (cpos - m.W);   // in [0, W + C)
          dst = b.part_win + (((size_t)s * b.nq + c) * m.R + off) * 128;
          const float a0 = m.scale * dk0[r], a1 = m.scale * dk1[r], a2 = dv0[r], a3 = dv1[r];
          if (q0 == 0) {
            dst[kl] = a0;
            dst[32 + kl] = a1;
            dst[64 + kl] = a2;
            dst[96 + kl] = a3;
          } else {
            dst[kl] += a0;
            dst[32 + kl] += a1;
            dst[64 + kl] += a2;
            dst[96 + kl] += a3;
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Window keys of one key block (the C positions [bC, bC + C)) against the
// query chunks whose window holds them (chunks b .. b + W/C): each wave keeps
// its key tile's dk and dv in registers across those chunks, and the block's
// final dk (RoPE transposed on dims 0..31, scaled) and dv are written once,
// with no partials in memory and no separate summing pass.  NW waves, wave w
// taking key tile w over all the chunk's 32-query sub-blocks; the chunk's
// queries and dO sit in LDS only as hi + lo query planes and dO in 128-byte
// rows with swizzled 16-byte units (~49 KB, so that two workgroups share a CU
// and one's staging overlaps the other's products): read directly as the
// score products' A operands and transposed (ds_read_b64_tr_b16) as the B
// operands of dk and dv.  The products are those of bwd_kv_mx_kernel's window
// tiles.
template <int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2))) void bwd_kvw_mx_kernel(
    Dims m, Dev d, BwdIn in, Bwd b) {
  constexpr int C = NW * 32;
  static_assert(C <= kQB, "one query block per chunk");
  constexpr int NV = NW;
  constexpr int QB = C;
  __shared__ __attribute__((aligned(16))) uint8_t Th[QB * 128];
  __shared__ __attribute__((aligned(16))) uint8_t Tl[QB * 128];
  __shared__ __attribute__((aligned(16))) uint8_t Td[QB * 128];
  __shared__ float2 LD[QB];
  const int s = blockIdx.x % m.BH;
  const int kb0 = blockIdx.x / m.BH;   // the key block
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, kl = lane & 31;
  const int tile = w;
  const int64_t bpos = (int64_t)kb0 * C;
  const int64_t kq = bpos + 32 * tile + kl;   // this lane's key
  const bool kvalid = kq < in.N;
  const int64_t pp = kvalid ? kq : in.N - 1;  // (a key past the end reads a valid row; masked)
  const int64_t klast = bpos + 32 * tile + 31;
  const float c2 = m.scale * kLog2e;
  const bf16* vin = reinterpret_cast<const bf16*>(in.v) + (size_t)s * in.N * 64;
  const bf16* doin = reinterpret_cast<const bf16*>(in.dout) + (size_t)s * in.N * 64;
  // this wave's keys (the rotated keys' hi plane) and values as B operands
  // (step kk: dims 16 kk + 8 h + e)
  bf16x8 kb[4], vb[4];
  {
    const bf16* kr = reinterpret_cast<const bf16*>(b.kr32) + ((size_t)s * in.N + pp) * 128;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      kb[kk] = *reinterpret_cast<const bf16x8*>(kr + 16 * kk + 8 * h);
      vb[kk] = *reinterpret_cast<const bf16x8*>(vin + pp * 64 + 16 * kk + 8 * h);
    }
  }
  f32x16 dk0 = {}, dk1 = {}, dv0 = {}, dv1 = {};
  const int c_end = min(kb0 + m.W / C, b.nq - 1);
  for (int c = kb0; c <= c_end; ++c) {
    const int64_t cpos = (int64_t)c * C;
    __syncthreads();   // every wave is done with the previous chunk's tiles
    // the chunk's queries, rotated (unscaled), their dO and (lse, D); zero past the end
    for (int e = tid; e < QB * 16; e += NV * 64) {
      const int qi = e >> 4, c4 = e & 15;
      const int64_t pos = cpos + qi;
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
      uint2 g = make_uint2(0u, 0u);
      if (pos < in.N) {
        x = *reinterpret_cast<const float4*>(b.qr32 + ((size_t)s * in.N + pos) * 64 + 4 * c4);
        g = *reinterpret_cast<const uint2*>(doin + pos * 64 + 4 * c4);
      }
      const bf16x4 h4{(bf16)x.x, (bf16)x.y, (bf16)x.z, (bf16)x.w};
      const bf16x4 l4{(bf16)(x.x - (float)h4[0]), (bf16)(x.y - (float)h4[1]), (bf16)(x.z - (float)h4[2]),
                      (bf16)(x.w - (float)h4[3])};
      const int o = qi * 128 + 16 * ((c4 >> 1) ^ tr_swz(qi)) + 8 * (c4 & 1);
      *reinterpret_cast<bf16x4*>(Th + o) = h4;
      *reinterpret_cast<bf16x4*>(Tl + o) = l4;
      *reinterpret_cast<uint2*>(Td + o) = g;
    }
    for (int qi = tid; qi < QB; qi += NV * 64) {
      const int64_t pos = cpos + qi;
      LD[qi] = pos < in.N ? b.lse_d[(size_t)s * in.N + pos] : make_float2(kInf, 0.f);
    }
    __syncthreads();
    // B operand of dk, dv at step kk: lane group g = lane / 16 reads queries
    // qs + 16 kk + 4 h + (lane % 16) / 4 (and + 8) at dims 32 half + 16 (g % 2) +
    // 4 (lane % 4); the transposed read hands lane l dim 32 half + l % 32
    auto qfrag = [&](const uint8_t* T, int qs, int kk, int half) __attribute__((always_inline)) {
      const int g = lane >> 4, pl = lane & 15;
      const int kq = 4 * h + (pl >> 2);
      const int d0 = 32 * half + 16 * (g & 1) + 4 * (pl & 3);
      const uint8_t* base = T + (qs + 16 * kk + kq) * 128 + 16 * ((d0 >> 3) ^ tr_swz(kq)) + 8 * ((d0 >> 2) & 1);
      const bf16x4 a = tr_read(base), c = tr_read(base + 8 * 128);
      return bf16x8{a[0], a[1], a[2], a[3], c[0], c[1], c[2], c[3]};
    };
    for (int j = 0; j < QB / 32; ++j) {
      const int qs = 32 * j;
      // S = Q . K^T and dP = dO . V^T, queries as rows (A operand rows qs + kl:
      // the 16-byte unit 2 kk + h of the row, swizzled)
      const uint8_t* qrow = Th + (qs + kl) * 128;
      const uint8_t* drow = Td + (qs + kl) * 128;
      f32x16 sc = {}, dp = {};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        sc = mfma_bf16(*reinterpret_cast<const bf16x8*>(qrow + 16 * ((2 * kk + h) ^ tr_swz(kl))), kb[kk], sc);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        dp = mfma_bf16(*reinterpret_cast<const bf16x8*>(drow + 16 * ((2 * kk + h) ^ tr_swz(kl))), vb[kk], dp);
      // (a query past the end has lse = +inf, so its weights come out 0; the
      // mask is needed only on a ragged tile or one with keys after some of
      // the sub-block's queries, i.e. in the key block's own chunk)
      f32x16 p, dsc;
      if (klast >= in.N || klast > cpos + qs) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qi = qs + mrow(r, h);
          const float2 ld = LD[qi];
          const bool ok = kvalid && kq <= cpos + qi;
          const float pr = ok ? exp2_fast(sc[r] * c2 - ld.x) : 0.f;
          p[r] = pr;
          dsc[r] = pr * (dp[r] - ld.y);
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float2 ld = LD[qs + mrow(r, h)];
          const float pr = exp2_fast(sc[r] * c2 - ld.x);
          p[r] = pr;
          dsc[r] = pr * (dp[r] - ld.y);
        }
      }
      // dk[key][d] += dS^T . Q (dS and Q as hi + lo pairs, three products) and
      // dv[key][e] += P^T . dO (P as a hi + lo pair, dO exact in bf16)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        float xa[8];
        bf16x8 dh, dl, ph, pl;
#pragma unroll
        for (int i = 0; i < 8; ++i) xa[i] = dsc[8 * kk + i];
        bf8_split(xa, dh, dl);
#pragma unroll
        for (int i = 0; i < 8; ++i) xa[i] = p[8 * kk + i];
        bf8_split(xa, ph, pl);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          f32x16& dk = half ? dk1 : dk0;
          f32x16& dv = half ? dv1 : dv0;
          const bf16x8 bh = qfrag(Th, qs, kk, half);
          const bf16x8 bl = qfrag(Tl, qs, kk, half);
          dk = mfma_bf16(dh, bh, dk);
          dk = mfma_bf16(dh, bl, dk);
          dk = mfma_bf16(dl, bh, dk);
          const bf16x8 od = qfrag(Td, qs, kk, half);
          dv = mfma_bf16(ph, od, dv);
          dv = mfma_bf16(pl, od, dv);
        }
      }
    }
  }
  // rows of the results are keys (register r: key mrow(r, h)), lane column =
  // dim; dk's dims 0..31 take RoPE transposed (partner dim kl ^ 16: the paired
  // row of 16 lanes)
  float* dko = b.dk + (size_t)s * in.N * 64;
  float* dvo = b.dv + (size_t)s * in.N * 64;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int64_t pos = bpos + 32 * tile + mrow(r, h);
    const float y = dk0[r];
    float ya, yb;
    row_pair(y, ya, yb);
    const float yp = (kl & 16) ? ya : yb;
    if (pos < in.N) {
      const int jf = kl & 15;
      const float cs = d.rope_cos[pos * 16 + jf], sn = d.rope_sin[pos * 16 + jf];
      const float x = kl < 16 ? y * cs + yp * sn : y * cs - yp * sn;
      dko[pos * 64 + kl] = m.scale * x;
      dko[pos * 64 + 32 + kl] = m.scale * dk1[r];
      dvo[pos * 64 + kl] = dv0[r];
      dvo[pos * 64 + 32 + kl] = dv1[r];
    }
  }
}

// ---------------------------------------------------------------------------
// Window keys: the partials of every chunk whose window holds position p (in
// chunk order), RoPE transposed on dims 0..31.  Writes dk and dv of every
// position (the state path adds to them later).  Sixteen threads per
// position, eight of the 128 partial columns each (dk 0..63, dv 64..127).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_win_kernel(Dims m, Dev d, BwdIn in, Bwd b) {
  const int s = blockIdx.y;
  const int64_t p0 = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int t = threadIdx.x & 15;
  const bool valid = p0 < in.N;
  const int64_t pos = valid ? p0 : in.N - 1;   // (every lane stays for the exchange below)
  const int64_t c0 = pos / m.C;
  int64_t c1 = (pos + m.W) / m.C;
  if (c1 > b.nq - 1) c1 = b.nq - 1;
  float g[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int64_t c = c0; c <= c1; ++c) {
    const int64_t off = pos - (c * m.C - m.W);
    const float* src = b.part_win + (((size_t)s * b.nq + c) * m.R + off) * 128 + 8 * t;
    const float4 a = *reinterpret_cast<const float4*>(src), e = *reinterpret_cast<const float4*>(src + 4);
    g[0] += a.x; g[1] += a.y; g[2] += a.z; g[3] += a.w;
    g[4] += e.x; g[5] += e.y; g[6] += e.z; g[7] += e.w;
  }
  // rotary dims (t < 4): the partner 16 dims away is thread t ^ 2 (a quad swap)
  float gp[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) gp[e] = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(g[e]), 0x4E, 0xF, 0xF, false));
  if (t < 4) {
    const float* cs = d.rope_cos + pos * 16 + ((8 * t) & 15);
    const float* sn = d.rope_sin + pos * 16 + ((8 * t) & 15);
    const float sg = t < 2 ? 1.f : -1.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) g[e] = fmaf(sg * gp[e], sn[e], g[e] * cs[e]);
  }
  if (valid) {
    float* dst = t < 8 ? b.dk + ((size_t)s * in.N + pos) * 64 + 8 * t : b.dv + ((size_t)s * in.N + pos) * 64 + 8 * (t - 8);
    *reinterpret_cast<float4*>(dst) = make_float4(g[0], g[1], g[2], g[3]);
    *reinterpret_cast<float4*>(dst + 4) = make_float4(g[4], g[5], g[6], g[7]);
  }
}

// ---------------------------------------------------------------------------
// State rows: for row i, from the last snapshot that holds it down to its
// creation, the read-form gradient of that snapshot's version is taken back to
// the raw sums (LayerNorm of K/n: dK = rs (g - mean g - x mean(g x)) / n; value
// rho u, u = V/|V|: dV = (rho/|V|) (g - u (u.g)), d rho = u.g; the plain mean
// V/n without value-length normalisation) and added to the running totals, which
// replace the partial in place: afterwards entry (j, i) holds the gradient of
// row i's sums as they stood after chunk j.  Four rows per wave, one per
// 16-lane row of the wave; lane q of a row holds key dims 2q, 2q + 1 and
// value dims 4q .. 4q + 3.
// ---------------------------------------------------------------------------
// Sums across lanes without LDS round trips, every lane receiving the sum (the
// same bits in every lane): DPP quad swaps and row mirrors within 16 lanes,
// then the row-pair and half-wave swaps.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_sum16(float v) {
  v += dpp_f<0xB1>(v);    // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);    // quad_perm [2,3,0,1]
  v += dpp_f<0x141>(v);   // row_half_mirror: the other quad of the 8
  v += dpp_f<0x140>(v);   // row_mirror: the other 8 of the row
  return v;
}
// sum over the lane's 32-lane half
__device__ __forceinline__ float lane_sum32(float v) {
  v = lane_sum16(v);
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float lane_sum64(float v) {
  v = lane_sum32(v);
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float2 ld2f(const float* p) { return *reinterpret_cast<const float2*>(p); }
typedef f16 f16x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float2 ld2f(const f16* p) {
  const f16x2v a = *reinterpret_cast<const f16x2v*>(p);
  return make_float2((float)a[0], (float)a[1]);
}
__device__ __forceinline__ float4 ld4f(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 ld4f(const bf16* p) {
  const bf16x4 a = *reinterpret_cast<const bf16x4*>(p);
  return make_float4((float)a[0], (float)a[1], (float)a[2], (float)a[3]);
}

template <typename T>
__global__ __launch_bounds__(256) void bwd_state_kernel(Dims m, Dev d, Bwd b, int rows_last) {
  using RT = typename Rd<T>::type;
  const int s = blockIdx.y;
  const int l = threadIdx.x & 63, q = l & 15;
  const int i0 = blockIdx.x * 16 + 4 * (threadIdx.x >> 6);
  if (i0 >= rows_last) return;   // (all four rows)
  const int i = i0 + (l >> 4);
  const bool row_ok = i < rows_last;
  const RT* pk = reinterpret_cast<const RT*>(d.pkey) + (size_t)s * m.V_cap * 32;
  const T* pv = reinterpret_cast<const T*>(d.pval) + (size_t)s * m.V_cap * 64;
  const float* prho = d.prho + (size_t)s * m.V_cap;
  const int* pcnt = d.pcount + (size_t)s * m.V_cap;
  const float2* pnm = d.pnorm + (size_t)s * m.V_cap;
  const int* idx = d.idx + (size_t)s * m.idx_total;
  float* part = b.part_state + (size_t)s * m.idx_total * 96;
  float* trho = b.tot_rho + (size_t)s * m.idx_total;
  float2 tk = make_float2(0.f, 0.f);
  float4 tv = make_float4(0.f, 0.f, 0.f, 0.f);
  float tr = 0.f;
  // The row's version id at snapshot j is loaded eight snapshots ahead of its
  // use and the version's inputs four ahead, so that neither waits on the
  // other.  Every fetch issues the same loads (at a valid index when the
  // snapshot or the row does not exist), so that the compiler's count of
  // loads in flight stays exact and each use waits for its own loads only.
  struct Id {
    int64_t off;
    int v0;
    bool live;
  };
  // The schedule, 64 chunks at a time in the wave's lanes (lane l: chunk
  // sb - l), read out with readlane: a load of the entry per snapshot would
  // sit between the loads in flight and their uses, and waiting for it would
  // wait for all of them.
  const int J = b.absorbed - 1;
  int sb = J, sS = 0, sW = 0;
  auto load_sched = [&](int top) {
    sb = top;
    const int jl = top - l;
    const int4 sc = d.sched[jl >= 0 ? jl : 0];
    sS = sc.x + sc.y + sc.z;
    sW = sc.w;
  };
  load_sched(J);
  auto fetch_id = [&](int j) {
    Id x;
    const int jc = j < 0 ? 0 : j;
    if (jc < sb - 63) load_sched(jc);   // (snapshots are visited in decreasing order)
    const int li = sb - jc;
    const int S = __builtin_amdgcn_readlane(sS, li), W = __builtin_amdgcn_readlane(sW, li);
    x.live = row_ok && j >= 0 && i < S;    // the row exists after chunk j
    x.off = (int64_t)W + i;      // inside the index lists either way
    x.v0 = idx[x.off];
    return x;
  };
  struct In {
    int64_t off;
    float2 gk, xh, nm;
    float4 gv, vh;
    float rho, invn;
    int ver;
    bool live;
  };
  // `nx` is the row at the next snapshot visited (j - 1).  The version's own
  // inputs are used only where a run of one version starts (the boundary
  // below); elsewhere the same loads read the pool's first version, which
  // stays in cache, so that only the boundaries fetch version data from HBM.
  auto fetch = [&](const Id& id, const Id& nx) {
    In x;
    x.live = id.live;
    x.off = id.off;
    x.ver = id.live ? id.v0 : 0;
    const int64_t ver = id.live && (!nx.live || nx.v0 != id.v0) ? id.v0 : 0;
    const float* e = part + x.off * 96;
    x.gk = ld2f(e + 2 * q);
    x.gv = ld4f(e + 32 + 4 * q);
    x.xh = ld2f(pk + ver * 32 + 2 * q);
    x.nm = pnm[ver];
    x.invn = __builtin_amdgcn_rcpf((float)pcnt[ver]);   // (1 ulp)
    x.rho = prho[ver];
    x.vh = ld4f(pv + ver * 64 + 4 * q);
    return x;
  };
  // Snapshots from the last down.  The LayerNorm and radius backward of a row
  // version is linear in the read-form gradient, and a row keeps its version
  // from the chunk that made it until the next that touches it, so the
  // snapshots' gradients are summed over each run of one version (G) and taken
  // back once, at the run's first snapshot: the chunk that touched the row (a
  // new version, or a new row; `prev` is the row at snapshot j - 1).  The
  // row's running total is stored there, the only snapshot whose total the
  // token pass reads back (the token that created or merged into the row).
  float2 Gk = make_float2(0.f, 0.f);
  float4 Gv = make_float4(0.f, 0.f, 0.f, 0.f);
  auto step = [&](const In& cur, const In& prev) {
    if (cur.live) {
      Gk.x += cur.gk.x;
      Gk.y += cur.gk.y;
      Gv.x += cur.gv.x;
      Gv.y += cur.gv.y;
      Gv.z += cur.gv.z;
      Gv.w += cur.gv.w;
    }
    const bool bnd = cur.live && (!prev.live || prev.ver != cur.ver);
    if (__any(bnd)) {   // (every lane takes part in the row sums; the others' results are unused)
      // LayerNorm backward over the 32 live dims (sums over the 16-lane row)
      const float sg = lane_sum16(Gk.x + Gk.y);
      const float sgx = lane_sum16(fmaf(Gk.y, cur.xh.y, Gk.x * cur.xh.x));
      const float ck = cur.nm.x * cur.invn;
      const float2 dK = make_float2(ck * (Gk.x - sg * (1.0f / 32.0f) - cur.xh.x * sgx * (1.0f / 32.0f)),
                                    ck * (Gk.y - sg * (1.0f / 32.0f) - cur.xh.y * sgx * (1.0f / 32.0f)));
      float4 dV;
      float dR = 0.f;
      if (m.no_vnorm) {
        dV = make_float4(Gv.x * cur.invn, Gv.y * cur.invn, Gv.z * cur.invn, Gv.w * cur.invn);
      } else {
        const float ir = cur.rho > 0.f ? __builtin_amdgcn_rcpf(cur.rho) : 0.f;   // (1 ulp)
        const float4 u = make_float4(cur.vh.x * ir, cur.vh.y * ir, cur.vh.z * ir, cur.vh.w * ir);
        const float ug = lane_sum16(fmaf(u.w, Gv.w, fmaf(u.z, Gv.z, fmaf(u.y, Gv.y, u.x * Gv.x))));
        const float cv = cur.nm.y;
        dV = make_float4(cv * (Gv.x - u.x * ug), cv * (Gv.y - u.y * ug), cv * (Gv.z - u.z * ug),
                         cv * (Gv.w - u.w * ug));
        dR = ug;
      }
      if (bnd) {
        tk.x += dK.x;
        tk.y += dK.y;
        tv.x += dV.x;
        tv.y += dV.y;
        tv.z += dV.z;
        tv.w += dV.w;
        tr += dR;
        float* e = part + cur.off * 96;
        *reinterpret_cast<float2*>(e + 2 * q) = tk;
        *reinterpret_cast<float4*>(e + 32 + 4 * q) = tv;
        if (q == 0) trho[cur.off] = tr;
        Gk = make_float2(0.f, 0.f);
        Gv = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
  };
  const Id c0 = fetch_id(J), c1 = fetch_id(J - 1), c2 = fetch_id(J - 2), c3 = fetch_id(J - 3);
  Id b0 = fetch_id(J - 4), b1 = fetch_id(J - 5), b2 = fetch_id(J - 6), b3 = fetch_id(J - 7);
  In a0 = fetch(c0, c1), a1 = fetch(c1, c2), a2 = fetch(c2, c3), a3 = fetch(c3, b0);
  for (int j = J; j >= 0; j -= 4) {
    // (a row exists from its creating chunk on, so the first snapshot without
    // it ends the sweep)
    if (!__any(a0.live)) break;
    step(a0, a1);
    a0 = fetch(b0, b1);
    b0 = fetch_id(j - 8);
    if (!__any(a1.live)) break;
    step(a1, a2);
    a1 = fetch(b1, b2);
    b1 = fetch_id(j - 9);
    if (!__any(a2.live)) break;
    step(a2, a3);
    a2 = fetch(b2, b3);
    b2 = fetch_id(j - 10);
    if (!__any(a3.live)) break;
    step(a3, a0);
    a3 = fetch(b3, b0);
    b3 = fetch_id(j - 11);
  }
}

// ---------------------------------------------------------------------------
// Absorbed tokens: a merged token added g * (k_live, v) to its row after its
// chunk; a sink or appended token created the row (k_live, v unscaled, radius
// |v|).  Adds to dk (live dims) and dv, writes the gate-logit gradient
// (sigmoid'), and zero for tokens never absorbed.  Sixteen threads per token
// (one DPP row): thread u holds value dims 4u .. 4u + 3 and, for u < 8, live
// key dims 32 + 4u .. + 3.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void load4f(const float* p, float (&x)[4]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
}
__device__ __forceinline__ void load4f(const bf16* p, float (&x)[4]) {
  const bf16x4 a = *reinterpret_cast<const bf16x4*>(p);
  x[0] = (float)a[0]; x[1] = (float)a[1]; x[2] = (float)a[2]; x[3] = (float)a[3];
}
template <typename T>
__global__ __launch_bounds__(256) void bwd_token_kernel(Dims m, Dev d, BwdIn in, Bwd b) {
  const int s = blockIdx.y;
  const int64_t t = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int u = threadIdx.x & 15;
  if (t >= in.N) return;   // (a whole row of sixteen leaves together)
  float* dl = b.dl + (size_t)s * in.N;
  if (t >= (int64_t)b.absorbed * m.C) {
    if (u == 0) dl[t] = 0.f;
    return;
  }
  const int j = (int)(t / m.C);
  const int kind = d.tkind[(size_t)s * m.max_tokens + t];
  const int row = d.tslot[(size_t)s * m.max_tokens + t];
  const int4 sc = d.sched[j];
  const int64_t off = (int64_t)s * m.idx_total + sc.w + row;
  const float* e = b.part_state + off * 96;
  const bool kl = u < 8;   // this thread also holds four live key dims
  const int ku = kl ? u : 0;
  float tk[4], tv[4], kt[4], vt[4];
  load4f(e + 4 * ku, tk);
  load4f(e + 32 + 4 * u, tv);
  const size_t ti = (size_t)s * in.N + (size_t)t;
  load4f(reinterpret_cast<const T*>(in.k) + ti * 64 + 32 + 4 * ku, kt);
  load4f(reinterpret_cast<const T*>(in.v) + ti * 64 + 4 * u, vt);
  float* dk = b.dk + ti * 64 + 32 + 4 * ku;
  float* dv = b.dv + ti * 64 + 4 * u;
  float ak[4], av[4];
  load4f(dk, ak);
  load4f(dv, av);
  if (kind == 2) {   // merge
    const float lg = in.l[ti];
    const float g = m.no_gate ? 1.f : 1.f / (1.f + __expf(-lg));
    float part = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (kl) part = fmaf(kt[q], tk[q], part);
      part = fmaf(vt[q], tv[q], part);
      ak[q] += g * tk[q];
      av[q] += g * tv[q];
    }
    const float dg = lane_sum16(part);
    if (u == 0) dl[t] = m.no_gate ? 0.f : dg * g * (1.f - g);
  } else {           // sink or append: the row's creator
    float part = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) part = fmaf(vt[q], vt[q], part);
    const float v2 = lane_sum16(part);
    const float tr = b.tot_rho[off];
    const float nv = sqrtf(v2);
    const float rs = nv > 0.f ? tr / nv : 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      ak[q] += tk[q];
      av[q] += tv[q] + rs * vt[q];
    }
    if (u == 0) dl[t] = 0.f;
  }
  if (kl) *reinterpret_cast<float4*>(dk) = make_float4(ak[0], ak[1], ak[2], ak[3]);
  *reinterpret_cast<float4*>(dv) = make_float4(av[0], av[1], av[2], av[3]);
}

template <typename T>
hipError_t bwd_dispatch(const Dims& m, const Dev& d, const BwdIn& in, const Bwd& b, int rows_last, hipStream_t st) {
  const dim3 grid((unsigned)(m.BH * b.nq));
  bwd_rot_kernel<T><<<dim3((unsigned)((in.N + 31) / 32), (unsigned)m.BH), 256, 0, st>>>(m, d, in, b);
  bool win_done = false;   // window-key gradients already written (no partials to sum)
  auto attn = [&](auto nw) {
    constexpr int NW = decltype(nw)::value;
    if constexpr (std::is_same<T, bf16>::value) {
      bwd_q_mx_kernel<NW><<<grid, NW * 64, 0, st>>>(m, d, in, b);
      constexpr int NV = NW < 8 ? 2 * NW : NW;
      if constexpr (NW < 8) {   // window keys in their own pass, no partials
        bwd_kv_mx_kernel<NW, NW, false><<<grid, NW * 64, 0, st>>>(m, d, in, b);
        bwd_kvw_mx_kernel<NW><<<grid, NW * 64, 0, st>>>(m, d, in, b);
        win_done = true;
      } else {
        bwd_kv_mx_kernel<NW, NV><<<grid, NV * 64, 0, st>>>(m, d, in, b);
      }
    } else {
      bwd_q_kernel<T, NW><<<grid, NW * 64, 0, st>>>(m, d, in, b);
      bwd_kv_kernel<T, NW><<<grid, NW * 64, 0, st>>>(m, d, in, b);
    }
  };
  switch (m.C) {
    case 32: attn(std::integral_constant<int, 1>{}); break;
    case 64: attn(std::integral_constant<int, 2>{}); break;
    case 128: attn(std::integral_constant<int, 4>{}); break;
    case 256: attn(std::integral_constant<int, 8>{}); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (!win_done) bwd_win_kernel<<<dim3((unsigned)((in.N + 15) / 16), (unsigned)m.BH), 256, 0, st>>>(m, d, in, b);
  if (rows_last > 0)
    bwd_state_kernel<T><<<dim3((unsigned)((rows_last + 15) / 16), (unsigned)m.BH), 256, 0, st>>>(m, d, b, rows_last);
  bwd_token_kernel<T><<<dim3((unsigned)((in.N + 15) / 16), (unsigned)m.BH), 256, 0, st>>>(m, d, in, b);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_backward(const Dims& m, const Dev& d, const BwdIn& in, const Bwd& b, int rows_last,
                           hipStream_t st) {
  if (in.N <= 0) return hipSuccess;
  return m.bf16 ? bwd_dispatch<bf16>(m, d, in, b, rows_last, st) : bwd_dispatch<float>(m, d, in, b, rows_last, st);
}

}  // namespace kvm
