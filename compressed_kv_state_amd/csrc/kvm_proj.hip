// gfx950 kernels of the projections around the Key-Value Means layer.
//
// [KVM abstract]: KVM is an attention layer, so a block feeds it queries, keys
// and values projected from the token representations and projects its output
// back; [KVM summary, Core mechanisms 2]: the merge gate is a data-dependent
// scalar, so its logit is one more projection of the same input, one per head.
//
// C[m][n] = sum_k A[m][k] W[n][k] (weights stored [out, in], both operands
// contiguous along k).  Two prologues / epilogues:
//   in-projection   A = x [B*N, D]; columns [0, D) q, [D, 2D) k, [2D, 3D) v
//                   (feature h*64 + d = dim d of head h) written to the layer's
//                   [B*H, N, 64] layout in the input type, [3D, 3D + H) the
//                   gate logits (+ per-head bias) as float32 [B*H, N];
//   out-projection  A gathered from the layer output o [B*H, N, 64] (row
//                   b*N + t, feature h*64 + d), C = y [B*N, D].
// bf16: 256 x 256 output tiles, eight waves of 128 x 64 (4 x 2 MFMA tiles of
// 32 x 32; two waves per SIMD), k in stages of 32 staged by direct
// global->LDS transfers, three stages in flight.
// fp32: 128 x 128 tiles, four waves of 64 x 64, k in stages of 32 through
// registers, double-buffered.
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


// ---------------------------------------------------------------------------
// bf16 GEMM.  A stage holds rows [256][64] of A and of W (128 bytes a row,
// eight 16-byte units, whole cache lines); the unit u of row r is stored at
// unit u ^ ((r >> 1) & 7), so that the 16 rows an MFMA operand read serves in
// one LDS cycle (same unit, consecutive rows) fall on distinct banks.  A
// global->LDS transfer writes 64 lanes x 16 bytes in lane order: lane l of
// transfer i fills row 8 i + l / 8, stored unit l % 8, and so fetches that
// row's unit (l % 8) ^ swizzle.
constexpr int kGM = 256, kGN = 256, kGK = 64;
constexpr int kGStageBytes = (kGM + kGN) * kGK * 2;   // 64 KB

__device__ __forceinline__ int gswz(int r) { return (r >> 1) & 7; }

template <bool OUT>
__global__ __launch_bounds__(512, 1) void proj_gemm_kernel(ProjArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t st0[kGStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t st1[kGStageBytes];
  // The accumulators are read only by the epilogue: naming one accumulation
  // register here lets the compiler keep them there, where the MFMA runs at
  // its full rate (measured: 34.6 against 42.9 cycles per 32x32x16 MFMA with
  // the accumulator in ordinary vector registers).
  asm volatile("" ::: "a0");
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w & 1, wn = w >> 1;   // wave tile: rows wm*128 + [0, 128), columns wn*64 + [0, 64)
  // tiles: dispatch b runs on XCD b mod 8.  With the row blocks a multiple of
  // 8, XCD x takes the row blocks = x (mod 8), in groups of four row blocks
  // swept across all column blocks, so that each row block of A and each
  // column block of W is fetched into that XCD's L2 once per group;
  // otherwise consecutive workgroups take the column blocks of one row block.
  const int n_nt = (a.Nout + kGN - 1) / kGN;
  const int m_nt = (int)((a.M + kGM - 1) / kGM);
  int mb, nb;
  if (m_nt % 8 == 0) {
    const int x = blockIdx.x & 7, k = blockIdx.x >> 3;
    constexpr int GM = 4;
    const int per = m_nt / 8;                    // row blocks of this XCD
    const int g = k / (GM * n_nt), r = k % (GM * n_nt);
    const int gm = min(GM, per - g * GM);        // row blocks in this group
    nb = r / gm;
    mb = 8 * (g * GM + r % gm) + x;
  } else {
    mb = blockIdx.x / n_nt;
    nb = blockIdx.x % n_nt;
  }
  const int64_t m0 = (int64_t)mb * kGM;
  const int n0 = nb * kGN;
  const bf16* X = reinterpret_cast<const bf16*>(a.x);
  const bf16* Wt = reinterpret_cast<const bf16*>(a.w);

  // this lane's four A rows and four W rows (transfers w + 8 i of each),
  // clamped to the last row (rows past the end are computed, not stored), and
  // the element offset of the unit it fetches
  const bf16* arow[4];
  const bf16* brow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 8 * (w + 8 * i) + (lane >> 3);
    const int ug = (lane & 7) ^ gswz(r);
    int64_t m = m0 + r;
    if (m > a.M - 1) m = a.M - 1;
    if constexpr (OUT) {
      const int64_t b = m / a.N, t = m % a.N;
      arow[i] = X + ((b * a.H) * a.N + t) * 64 + 8 * ug;   // head 0; stage k0 adds head k0/64
    } else {
      arow[i] = X + m * a.K + 8 * ug;
    }
    int n = n0 + r;
    if (n > a.Nout - 1) n = a.Nout - 1;
    brow[i] = Wt + (int64_t)n * a.K + 8 * ug;
  }
  auto issue = [&](int k0, uint8_t* stg) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16* src;
      if constexpr (OUT) src = arow[i] + (int64_t)(k0 >> 6) * a.N * 64;   // the stage is one head's 64 dims
      else src = arow[i] + k0;
      __builtin_amdgcn_global_load_lds(src, stg + 1024 * (w + 8 * i), 16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_global_load_lds(brow[i] + k0, stg + kGM * 128 + 1024 * (w + 8 * i), 16, 0, 0);
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  // MFMA operand reads: A rows wm*128 + 32 i + lane % 32, W rows wn*64 + 32 j + lane % 32,
  // unit 2 ks + h of the stage's 64 k.  The swizzle of those rows depends on
  // the lane only, so each read is a per-lane offset (one per ks) plus a constant.
  int offa[4], offb[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int u = 16 * ((2 * ks + h) ^ gswz(l32));
    offa[ks] = (wm * 128 + l32) * 128 + u;
    offb[ks] = kGM * 128 + (wn * 64 + l32) * 128 + u;
  }
  auto compute = [&](const uint8_t* stg) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8 af[4], bfr[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) af[i] = *reinterpret_cast<const bf16x8*>(stg + offa[ks] + 4096 * i);
#pragma unroll
      for (int j = 0; j < 2; ++j) bfr[j] = *reinterpret_cast<const bf16x8*>(stg + offb[ks] + 4096 * j);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma_bf16(af[i], bfr[j], acc[i][j]);
    }
  };

  // two stages: each barrier follows the wave's wait for its own transfers of
  // the stage about to be computed; the transfer of the next stage overlaps it.
  // (Separate buffers, unrolled by two with one exit, so that the compiler sees
  // which buffer each read and transfer touches and keeps the accumulators put.)
  // (The scheduling barriers keep each stage's transfers ahead of the other
  // stage's products: left free, the compiler sinks them to the end of the
  // products, right before the wait for them, and nothing overlaps.)
  const int nk = a.K / kGK;
  issue(0, st0);
  int kt = 0;
  for (; kt + 2 <= nk; kt += 2) {
    dma_barrier();
    issue((kt + 1) * kGK, st1);
    __builtin_amdgcn_sched_barrier(0);
    compute(st0);
    dma_barrier();
    if (kt + 2 < nk) issue((kt + 2) * kGK, st0);
    __builtin_amdgcn_sched_barrier(0);
    compute(st1);
  }
  if (kt < nk) {   // an odd last stage, in flight in the first buffer
    dma_barrier();
    compute(st0);
  }

  // epilogue: register r of a 32 x 32 tile is row 8(r/4) + 4h + r%4, column
  // lane % 32.  Destinations split into a row part and a column part: the
  // row parts of the tile's 256 rows go to LDS first (one division per row).
  //   in:  q/k/v element ((b H + f/64) N + t) 64 + f%64 = rowq(m) + colq(n),
  //        rowq = (b H N + t) 64, colq = (f/64) N 64 + f%64;
  //        gate logit (b H + hh) N + t = rowg(m) + hh N, rowg = b H N + t;
  //   out: y element m Nout + n.
  // A wave's 64 columns are 64-aligned, so they lie in one destination part
  // and, for q/k/v, in one head: the bf16 parts go through LDS (the wave's
  // 128 x 64 tile, 16-byte units XOR-swizzled by row) and leave as 16-byte
  // stores of eight consecutive columns; the fp32 gate logits are stored one
  // by one.
  __shared__ int64_t rowpart[kGM];
  __syncthreads();   // every wave is done with the stages
  if constexpr (!OUT) {
    if (tid < kGM) {
      int64_t m = m0 + tid;
      if (m > a.M - 1) m = a.M - 1;
      const int64_t b = m / a.N, t = m % a.N;
      rowpart[tid] = b * a.H * a.N + t;
    }
  }
  const int D = a.H * 64;
  const int nw0 = n0 + wn * 64;                 // the wave's first column
  const bool gate = !OUT && nw0 >= 3 * D;       // gate-logit columns (fp32)
  uint8_t* tile = (w < 4 ? st0 : st1) + (w & 3) * (128 * 128);
  if (!gate) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = 32 * i + 8 * (r >> 2) + 4 * h + (r & 3), col = 32 * j + l32;
          *reinterpret_cast<bf16*>(tile + row * 128 + (((col >> 3) ^ (row & 7)) << 4) + (col & 7) * 2) =
              (bf16)acc[i][j][r];
        }
  }
  __syncthreads();   // row parts (and each wave's own tile) visible
  if (!gate) {
    const int part = OUT ? 0 : nw0 / D;
    bf16* dst = OUT ? reinterpret_cast<bf16*>(a.y)
                    : reinterpret_cast<bf16*>(part == 0 ? a.q : (part == 1 ? a.k : a.v));
#pragma unroll
    for (int it = 0; it < 16; ++it) {
      const int row = 8 * it + (lane >> 3), u = lane & 7;
      const int rl = wm * 128 + row;
      const int64_t m = m0 + rl;
      const int n = nw0 + 8 * u;
      if (m >= a.M || n >= a.Nout) continue;
      const uint4 v = *reinterpret_cast<const uint4*>(tile + row * 128 + ((u ^ (row & 7)) << 4));
      int64_t off;
      if constexpr (OUT) {
        off = m * a.Nout + n;
      } else {
        const int f = n - part * D;
        off = rowpart[rl] * 64 + (int64_t)(f >> 6) * a.N * 64 + (f & 63);
      }
      *reinterpret_cast<uint4*>(dst + off) = v;
    }
  } else {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = nw0 + 32 * j + l32;
      if (n >= a.Nout) continue;
      const int64_t col = (int64_t)(n - 3 * D) * a.N;
      const float bv = a.bias ? a.bias[n - 3 * D] : 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rl = wm * 128 + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
          if (m0 + rl >= a.M) continue;
          a.gl[rowpart[rl] + col] = acc[i][j][r] + bv;
        }
    }
  }
}

}  // namespace

hipError_t launch_proj(const ProjArgs& a, bool out, bool is_bf16, hipStream_t st) {
  if (a.M <= 0) return hipSuccess;
  const unsigned grid = (unsigned)(((a.M + kPM - 1) / kPM) * ((a.Nout + kPN - 1) / kPN));
  if (is_bf16) {
    const unsigned g = (unsigned)(((a.M + kGM - 1) / kGM) * ((a.Nout + kGN - 1) / kGN));
    if (out) proj_gemm_kernel<true><<<g, 512, 0, st>>>(a);
    else proj_gemm_kernel<false><<<g, 512, 0, st>>>(a);
  } else {
    if (out) proj_kernel<float, true><<<grid, 256, 0, st>>>(a);
    else proj_kernel<float, false><<<grid, 256, 0, st>>>(a);
  }
  return hipGetLastError();
}

}  // namespace kvm
