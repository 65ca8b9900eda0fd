// Finalize: weighted un-permute and sum, identity experts, residual.
//
// [P1] "Qwen3-MoE low-latency inference on Atlas A3 / 950 clusters",
// section 高效排序和token路由: finalize_routing puts the expert outputs back in
// token order and takes their weighted sum. [P2] "LongCat-Flash inference on
// Atlas A3 clusters", MoE模块 / Decode阶段优化: a zero-compute expert returns
// its input, MoE(x) = x.
//
// One block per token. The token's k slots are resolved once (into LDS) to
// a source row: its expert output row in y, its own x row for an identity
// expert, or nothing for an expert outside [lb, le); the slots that add
// something are compacted in slot order. Each thread owns 8 consecutive
// columns (16 bytes of bf16), loads the rows of 8 kept slots at a time and
// sums in fp32 from the residual, in slot order j = 0..k-1, then rounds once.
#include "common.h"
#include "launch.h"

namespace moe {

template <int ACT>
MOE_DEV void load8(const void* base, size_t row, int H, int c, float f[8]) {
  if (ACT == 0) {
    const float4* p = (const float4*)((const float*)base + row * H) + 2 * c;
    float4 a = p[0], b = p[1];
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  } else {
    uint4 v = ((const uint4*)((const uint16_t*)base + row * H))[c];
    f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x); f[2] = bf16_lo(v.y);
    f[3] = bf16_hi(v.y); f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
    f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
  }
}

// Source row of each of a token's k slots, decided once per token: a row of
// y (>= 0), the token's own x row (kIdentity) or nothing (kDropped).
constexpr int kIdentity = -1, kDropped = -2;
constexpr int kMaxSlots = 64;
constexpr int kBatch = 8;  // slots whose rows are loaded together

template <int ACT>
__global__ __launch_bounds__(256) void finalize_kernel(
    const int32_t* __restrict__ ids, const float* __restrict__ wts,
    const int32_t* __restrict__ copy_pos, const int32_t* __restrict__ offsets,
    int fb, int n_ffn, int lb, int le, const void* __restrict__ y,
    const void* __restrict__ x, const void* __restrict__ residual,
    void* __restrict__ out, int H, int k) {
  __shared__ int32_t s_row[kMaxSlots];
  __shared__ float s_w[kMaxSlots];
  __shared__ int32_t s_n;
  const int t = blockIdx.x;
  // wave 0 keeps the slots that add something, in slot order (k <= 64)
  if (threadIdx.x < 64) {
    const int j = threadIdx.x;
    int row = kDropped;
    float wj = 0.f;
    if (j < k) {
      const int e = ids[t * k + j];
      if (e >= lb && e < le)
        row = e >= n_ffn ? kIdentity : copy_pos[t * k + j] - offsets[fb];
      wj = wts[t * k + j];
    }
    const uint64_t keep = ballot(row != kDropped);
    if (row != kDropped) {
      const int pos = popc64(keep & lanemask_lt());
      s_row[pos] = row;
      s_w[pos] = wj;
    }
    if (j == 0) s_n = popc64(keep);
  }
  __syncthreads();
  const int n = s_n;
  for (int c = threadIdx.x; c < H / 8; c += blockDim.x) {
    float acc[8];
    if (residual) {
      load8<ACT>(residual, t, H, c, acc);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    }
    for (int j0 = 0; j0 < n; j0 += kBatch) {
      // rows of up to kBatch kept slots in flight together (entries past n
      // re-read the first kept row and are not added), then the fp32 sum in
      // slot order
      float v[kBatch][8];
#pragma unroll
      for (int jj = 0; jj < kBatch; ++jj) {
        const int j = j0 + jj;
        const int row = s_row[j < n ? j : 0];
        const bool from_y = row >= 0;
        load8<ACT>(from_y ? y : x, from_y ? (size_t)row : (size_t)t, H, c,
                   v[jj]);
      }
#pragma unroll
      for (int jj = 0; jj < kBatch; ++jj) {
        if (j0 + jj < n) {
          const float wj = s_w[j0 + jj];
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] = fmaf(wj, v[jj][i], acc[i]);
        }
      }
    }
    if (ACT == 0) {
      float4* p = (float4*)((float*)out + (size_t)t * H) + 2 * c;
      p[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
      p[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    } else {
      uint4 o;
      o.x = pack_bf16x2(acc[0], acc[1]);
      o.y = pack_bf16x2(acc[2], acc[3]);
      o.z = pack_bf16x2(acc[4], acc[5]);
      o.w = pack_bf16x2(acc[6], acc[7]);
      ((uint4*)((uint16_t*)out + (size_t)t * H))[c] = o;
    }
  }
}

hipError_t launch_finalize(const int32_t* ids, const float* w,
                           const int32_t* copy_pos, const int32_t* offsets,
                           int fb, int n_ffn, int lb, int le, const void* y,
                           const void* x, const void* residual, void* out,
                           int act, int T, int H, int k, hipStream_t s) {
  if (T == 0) return hipSuccess;
  int threads = H / 8 < 256 ? ((H / 8 + 63) / 64) * 64 : 256;
  if (act == 0)
    hipLaunchKernelGGL(finalize_kernel<0>, dim3(T), dim3(threads), 0, s, ids,
                       w, copy_pos, offsets, fb, n_ffn, lb, le, y, x, residual,
                       out, H, k);
  else
    hipLaunchKernelGGL(finalize_kernel<1>, dim3(T), dim3(threads), 0, s, ids,
                       w, copy_pos, offsets, fb, n_ffn, lb, le, y, x, residual,
                       out, H, k);
  return hipGetLastError();
}

}  // namespace moe
