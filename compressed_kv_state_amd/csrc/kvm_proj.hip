// gfx950 kernels of the projections around the Key-Value Means layer.
//
// [KVM abstract]: KVM is an attention layer, so a block feeds it queries, keys
// and values projected from the token representations and projects its output
// back; [KVM summary, Core mechanisms 2]: the merge gate is a data-dependent
// scalar, so its logit is one more projection of the same input, one per head.
//
// One GEMM kernel, C[m][n] = sum_k A[m][k] W[n][k] (weights stored [out, in],
// both operands contiguous along k), 128 x 128 output tiles, four waves of 64 x 64
// (2 x 2 MFMA tiles of 32 x 32), k in stages of 64 (bf16, v_mfma_f32_32x32x16_bf16)
// or 32 (fp32, v_mfma_f32_32x32x2f32), double-buffered through LDS, with the
// next stage's global loads in flight during the current stage's products.
// Two epilogues / prologues:
//   in-projection   A = x [B*N, D]; columns [0, D) q, [D, 2D) k, [2D, 3D) v
//                   (feature h*64 + d = dim d of head h) written to the layer's
//                   [B*H, N, 64] layout in the input type, [3D, 3D + H) the
//                   gate logits (+ per-head bias) as float32 [B*H, N];
//   out-projection  A gathered from the layer output o [B*H, N, 64] (row
//                   b*N + t, feature h*64 + d), C = y [B*N, D].
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvm_device.h"
#include "kvm_internal.h"

namespace kvm {
namespace {

template <typename T> struct ProjGeom;
template <> struct ProjGeom<bf16> {
  static constexpr int BK = 64;      // k per stage
  static constexpr int PITCH = 72;   // LDS row pitch (elements): 144 B, 16 lanes' 16-byte reads on distinct banks
};
template <> struct ProjGeom<float> {
  static constexpr int BK = 32;
  static constexpr int PITCH = 33;   // odd: 32 rows at one column land on distinct banks
};

constexpr int kPM = 128, kPN = 128;   // output tile

template <typename T, bool OUT>
__global__ __launch_bounds__(256, 2) void proj_kernel(ProjArgs a) {
  constexpr int BK = ProjGeom<T>::BK, PITCH = ProjGeom<T>::PITCH;
  constexpr int EPC = 16 / (int)sizeof(T);    // elements per 16-byte chunk
  constexpr int CPR = BK / EPC;               // chunks per tile row and stage (8)
  constexpr int LOADS = kPM * CPR / 256;      // chunks per thread and operand (4)
  __shared__ __attribute__((aligned(16))) T As[2][kPM * PITCH];
  __shared__ __attribute__((aligned(16))) T Bs[2][kPN * PITCH];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, l32 = lane & 31;
  const int wm = w >> 1, wn = w & 1;
  // tile order: consecutive workgroups share the same weight columns (n tile) so
  // that the weights stay in L2 while the token tiles stream
  const int n_mt = (int)((a.M + kPM - 1) / kPM);
  const int64_t m0 = (int64_t)(blockIdx.x % n_mt) * kPM;
  const int n0 = (int)(blockIdx.x / n_mt) * kPN;
  const T* Wt = reinterpret_cast<const T*>(a.w);

  // global addresses of this thread's chunks (row clamped: rows past the end are computed, not stored)
  const T* asrc[LOADS];
  const T* bsrc[LOADS];
  int arow[LOADS], akc[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int c = tid + 256 * i;
    arow[i] = c / CPR;
    akc[i] = c % CPR;
    int64_t m = m0 + arow[i];
    if (m > a.M - 1) m = a.M - 1;
    if constexpr (OUT) {
      const int64_t b = m / a.N, t = m % a.N;
      // row b*N + t of the gathered A, head h at k = h*64 + d: o[(b*H + h)*N + t][d]
      asrc[i] = reinterpret_cast<const T*>(a.x) + ((b * a.H) * a.N + t) * 64 + akc[i] * EPC;
    } else {
      asrc[i] = reinterpret_cast<const T*>(a.x) + m * a.K + akc[i] * EPC;
    }
    int n = n0 + arow[i];
    if (n > a.Nout - 1) n = a.Nout - 1;
    bsrc[i] = Wt + (int64_t)n * a.K + akc[i] * EPC;
  }
  uint4 ar[LOADS], br[LOADS];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      if constexpr (OUT) {
        // stage k0 lies in head k0/64, dims k0%64 ...: that head's row of o
        const int64_t hoff = (int64_t)(k0 / 64) * a.N * 64 + (k0 % 64);
        ar[i] = *reinterpret_cast<const uint4*>(asrc[i] + hoff);
      } else {
        ar[i] = *reinterpret_cast<const uint4*>(asrc[i] + k0);
      }
      br[i] = *reinterpret_cast<const uint4*>(bsrc[i] + k0);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      T* ad = &As[buf][arow[i] * PITCH + akc[i] * EPC];
      T* bd = &Bs[buf][arow[i] * PITCH + akc[i] * EPC];
      if constexpr (sizeof(T) == 2) {
        *reinterpret_cast<uint4*>(ad) = ar[i];
        *reinterpret_cast<uint4*>(bd) = br[i];
      } else {
        const float* af = reinterpret_cast<const float*>(&ar[i]);
        const float* bf = reinterpret_cast<const float*>(&br[i]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ad[e] = af[e];
          bd[e] = bf[e];
        }
      }
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) acc[mi][ni] = f32x16{};

  const int stages = (int)(a.K / BK);
  gload(0);
  lstore(0);
  __syncthreads();
  for (int st = 0; st < stages; ++st) {
    const int buf = st & 1;
    if (st + 1 < stages) gload((st + 1) * BK);
    const T* Ab = As[buf];
    const T* Bb = Bs[buf];
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        bf16x8 af[2], bfr[2];
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
          af[mi] = *reinterpret_cast<const bf16x8*>(Ab + (wm * 64 + mi * 32 + l32) * PITCH + ks * 16 + 8 * h);
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          bfr[ni] = *reinterpret_cast<const bf16x8*>(Bb + (wn * 64 + ni * 32 + l32) * PITCH + ks * 16 + 8 * h);
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
          for (int ni = 0; ni < 2; ++ni) acc[mi][ni] = mfma_bf16(af[mi], bfr[ni], acc[mi][ni]);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < BK / 2; ++ks) {
        float af[2], bfr[2];
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) af[mi] = Ab[(wm * 64 + mi * 32 + l32) * PITCH + 2 * ks + h];
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) bfr[ni] = Bb[(wn * 64 + ni * 32 + l32) * PITCH + 2 * ks + h];
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
          for (int ni = 0; ni < 2; ++ni) acc[mi][ni] = mfma_f32(af[mi], bfr[ni], acc[mi][ni]);
      }
    }
    if (st + 1 < stages) lstore(buf ^ 1);
    __syncthreads();
  }

  // epilogue: register r of a 32 x 32 tile is row 8(r/4) + 4h + r%4, column lane % 32
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
      const int n = n0 + wn * 64 + ni * 32 + l32;
      if (n >= a.Nout) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm * 64 + mi * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        if (m >= a.M) continue;
        const float val = acc[mi][ni][r];
        if constexpr (OUT) {
          reinterpret_cast<T*>(a.y)[m * a.Nout + n] = fromf<T>(val);
        } else {
          const int64_t b = m / a.N, t = m % a.N;
          const int D = a.H * 64;
          if (n < 3 * D) {
            const int part = n / D, f = n % D;
            T* dst = reinterpret_cast<T*>(part == 0 ? a.q : (part == 1 ? a.k : a.v));
            dst[((b * a.H + f / 64) * a.N + t) * 64 + (f & 63)] = fromf<T>(val);
          } else {
            const int hh = n - 3 * D;
            a.gl[(b * a.H + hh) * a.N + t] = val + (a.bias ? a.bias[hh] : 0.f);
          }
        }
      }
    }
}

}  // namespace

hipError_t launch_proj(const ProjArgs& a, bool out, bool is_bf16, hipStream_t st) {
  if (a.M <= 0) return hipSuccess;
  const unsigned grid = (unsigned)(((a.M + kPM - 1) / kPM) * ((a.Nout + kPN - 1) / kPN));
  if (is_bf16) {
    if (out) proj_kernel<bf16, true><<<grid, 256, 0, st>>>(a);
    else proj_kernel<bf16, false><<<grid, 256, 0, st>>>(a);
  } else {
    if (out) proj_kernel<float, true><<<grid, 256, 0, st>>>(a);
    else proj_kernel<float, false><<<grid, 256, 0, st>>>(a);
  }
  return hipGetLastError();
}

}  // namespace kvm
