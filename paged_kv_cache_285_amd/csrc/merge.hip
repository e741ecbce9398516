// Merge of attention states over disjoint key sets [2048ai.net vLLM V1 article, "Cascade
// Inference": the prefix state and the suffix state are combined by an associative and
// commutative merge operator].  With Z = e^lse, the union's state is
// o = (Z_a o_a + Z_b o_b) / (Z_a + Z_b), lse = ln(Z_a + Z_b); evaluated shifted by the larger
// lse so nothing overflows, and (0, -inf) acts as the identity.
#include "internal.h"

namespace pkv {
namespace {

// One thread per 4 consecutive output elements of one (token, head) row.
__global__ void merge_kernel(void* __restrict__ out, int32_t out_f32, float* __restrict__ lse_out,
                             const float4* __restrict__ oa, const float* __restrict__ la,
                             const float4* __restrict__ ob, const float* __restrict__ lb,
                             int64_t rows, int32_t vec_per_row) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = gid / vec_per_row;
  if (row >= rows) return;
  const int32_t c = (int32_t)(gid - row * vec_per_row);
  const float a = la[row], b = lb[row];
  const float m = fmaxf(a, b);
  float wa = 0.f, wb = 0.f, lse = -INFINITY;
  if (m != -INFINITY) {
    wa = (a == -INFINITY) ? 0.f : __expf(a - m);
    wb = (b == -INFINITY) ? 0.f : __expf(b - m);
    const float z = wa + wb;
    lse = m + __logf(z);
    const float inv = 1.f / z;
    wa *= inv;
    wb *= inv;
  }
  const float4 x = oa[gid], y = ob[gid];
  float4 r;
  r.x = wa * x.x + wb * y.x;
  r.y = wa * x.y + wb * y.y;
  r.z = wa * x.z + wb * y.z;
  r.w = wa * x.w + wb * y.w;
  if (m == -INFINITY) r = make_float4(0.f, 0.f, 0.f, 0.f);
  if (out_f32) {
    reinterpret_cast<float4*>(out)[gid] = r;
  } else {
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    bf16x4 h = {(__bf16)r.x, (__bf16)r.y, (__bf16)r.z, (__bf16)r.w};
    reinterpret_cast<bf16x4*>(out)[gid] = h;
  }
  if (lse_out && c == 0) lse_out[row] = lse;
}

}  // namespace

hipError_t launch_merge(void* out, int32_t out_f32, float* lse_out, const float* oa,
                        const float* la, const float* ob, const float* lb, int64_t rows,
                        int32_t head_dim, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const int32_t vec = head_dim / 4;
  const int64_t total = rows * vec;
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream, out, out_f32,
                     lse_out, reinterpret_cast<const float4*>(oa), la,
                     reinterpret_cast<const float4*>(ob), lb, rows, vec);
  return hipGetLastError();
}

}  // namespace pkv
