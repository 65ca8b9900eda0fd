// fp32 router linear in front of the gate: logits = y @ w_router^T.
//
// [P1] "Qwen3-MoE low-latency inference on Atlas A3 / 950 clusters", section
// 融合算子优化 / 融合RMSNorm Cast: the norm in front of the MoE block emits fp32
// hidden states for the gate (router) computation and bf16 ones for the
// experts. The router is a linear map without bias, one logit per expert.
//
// y [T, H] and w_router [E, H] are both K-contiguous fp32. A block owns 32
// tokens x 64 experts (16 x 32 for small shapes); its KS waves split H and
// add their partial sums in LDS. v_mfma_f32_16x16x4_f32: lane l holds row (A) / column (B) l%16 at
// K = l/16. Each lane loads four consecutive K (16 bytes) of each of its
// token and expert rows per 16-K step and feeds element i of each to the
// i-th of four MFMAs; A and B lanes hold the same K, so the four MFMAs
// together sum the step's 16 K. fp32 accumulation throughout.
#include "common.h"
#include "launch.h"

namespace moe {

namespace {

MOE_DEV f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// MB x NB blocks of 16 x 16 per wave (MB token blocks, NB expert blocks)
template <int KS, int MB, int NB>
__global__ __launch_bounds__(64 * KS) void router_logits_kernel(
    const float* __restrict__ y, const float* __restrict__ w,
    float* __restrict__ out, int T, int H, int E) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane & 15, q = lane >> 4;
  const int t0 = blockIdx.x * 16 * MB, e0 = blockIdx.y * 16 * NB;
  const float* yr[MB];
  const float* wr[NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    // token rows past T read row T-1 (their outputs are not stored)
    const int tr = min(t0 + 16 * mb + g, T - 1);
    yr[mb] = y + (size_t)tr * H + 4 * q;
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
    wr[nb] = w + (size_t)(e0 + 16 * nb + g) * H + 4 * q;
  const int nsteps = H / 16;
  const int s0 = wave * nsteps / KS, s1 = (wave + 1) * nsteps / KS;
  f32x4 acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  // a ring of D register stages: the loads of the next D-1 steps are in
  // flight while a step is multiplied (the last steps reload the final step,
  // harmlessly, instead of branching)
  constexpr int D = 3;
  float4 a[D][MB], b[D][NB];
  auto load = [&](int i, int st) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) a[i][mb] = *(const float4*)(yr[mb] + 16 * st);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) b[i][nb] = *(const float4*)(wr[nb] + 16 * st);
  };
  if (s0 < s1) {
#pragma unroll
    for (int i = 0; i < D; ++i) load(i, min(s0 + i, s1 - 1));
  }
  for (int s = s0; s < s1; s += D) {
#pragma unroll
    for (int i = 0; i < D; ++i) {
      if (s + i < s1) {
        // MB x NB independent accumulators: consecutive MFMAs never chain
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
              acc[mb][nb] = mfma_f32(a[i][mb][c], b[i][nb][c], acc[mb][nb]);
        load(i, min(s + i + D, s1 - 1));
      }
    }
  }
  if (KS > 1) {
    constexpr int NR = MB * NB * 4;
    __shared__ float red[(KS > 1 ? KS - 1 : 1) * NR * 64];
    if (wave > 0) {
#pragma unroll
      for (int x = 0; x < NR; ++x)
        red[((wave - 1) * NR + x) * 64 + lane] = acc[x / (NB * 4)][(x / 4) % NB][x % 4];
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int ww = 0; ww < KS - 1; ++ww)
#pragma unroll
      for (int x = 0; x < NR; ++x)
        acc[x / (NB * 4)][(x / 4) % NB][x % 4] += red[(ww * NR + x) * 64 + lane];
  }
  // lane holds rows t0 + 16*mb + 4q + r of columns e0 + 16*nb + g
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = t0 + 16 * mb + 4 * q + r;
      if (t < T) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          out[(size_t)t * E + e0 + 16 * nb + g] = acc[mb][nb][r];
      }
    }
}

}  // namespace

template <int MB, int NB>
static hipError_t launch_rl(const float* y, const float* w, float* out, int T,
                            int H, int E, hipStream_t s) {
  const dim3 grid((unsigned)((T + 16 * MB - 1) / (16 * MB)),
                  (unsigned)(E / (16 * NB)));
  // waves per block that split H: fill about four waves per SIMD, keep at
  // least four 16-K steps per wave
  const long long tiles = (long long)grid.x * grid.y;
  const long long slots = (long long)device_cus() * 16;
  int ks = 1;
  while (ks < 8 && tiles * ks * 2 <= slots && H / 16 / (ks * 2) >= 4) ks *= 2;
  switch (ks) {
    case 1:
      hipLaunchKernelGGL((router_logits_kernel<1, MB, NB>), grid, dim3(64), 0,
                         s, y, w, out, T, H, E);
      break;
    case 2:
      hipLaunchKernelGGL((router_logits_kernel<2, MB, NB>), grid, dim3(128), 0,
                         s, y, w, out, T, H, E);
      break;
    case 4:
      hipLaunchKernelGGL((router_logits_kernel<4, MB, NB>), grid, dim3(256), 0,
                         s, y, w, out, T, H, E);
      break;
    default:
      hipLaunchKernelGGL((router_logits_kernel<8, MB, NB>), grid, dim3(512), 0,
                         s, y, w, out, T, H, E);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_router_logits(const float* y, const float* w, float* out,
                                int T, int H, int E, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  // 32 tokens x 64 experts per wave (a load feeds 4 to 8 MFMAs) for
  // prefill-size batches; small batches take 16 x 32 wave tiles, four times
  // as many waves (measured at T = 32: 17.7 against 30 us)
  if (E % 64 == 0 && T >= 256) return launch_rl<2, 4>(y, w, out, T, H, E, s);
  return launch_rl<1, 2>(y, w, out, T, H, E, s);
}

}  // namespace moe
