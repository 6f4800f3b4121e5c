// Log-sum-exp merge of attention parts over the same queries (NanoKV, Figure 4d:
// parts of the history attended separately are combined by LSE merging).
//   L = m + ln sum_p exp(L_p - m),  m = max_p L_p;   O = sum_p exp(L_p - L) O_p.
// Parts with L_p = -inf carry no weight; all parts -inf gives O = 0, L = -inf.
#include "kvc_internal.h"

namespace kvc {
namespace {

struct PartPtrs {
  const float* o[kMaxMergeParts];
  const float* l[kMaxMergeParts];
};

// One thread per (row, 4 output channels).  Each thread reads the P row LSEs and
// forms the weights itself; the output is written after every input is read, so
// out/lse may alias part 0.
__global__ __launch_bounds__(256) void lse_merge_kernel(PartPtrs parts, int n_parts, int64_t rows, int dim4,
                                                         float* __restrict__ out, float* __restrict__ lse) {
  const int64_t item = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (item >= rows * dim4) return;
  const int64_t row = item / dim4;
  const int c4 = int(item % dim4);
  float m = -INFINITY;
  for (int p = 0; p < n_parts; ++p) m = fmaxf(m, parts.l[p][row]);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float L = -INFINITY;
  if (m != -INFINITY) {
    float tot = 0.f;
    for (int p = 0; p < n_parts; ++p) tot += expf(parts.l[p][row] - m);
    L = m + logf(tot);
    for (int p = 0; p < n_parts; ++p) {
      const float w = expf(parts.l[p][row] - L);
      const float4 o = reinterpret_cast<const float4*>(parts.o[p] + row * int64_t(dim4) * 4)[c4];
      acc.x += w * o.x; acc.y += w * o.y; acc.z += w * o.z; acc.w += w * o.w;
    }
  }
  __syncthreads();  // keeps every read of this block before any write (aliasing of part 0)
  reinterpret_cast<float4*>(out + row * int64_t(dim4) * 4)[c4] = acc;
  if (c4 == 0) lse[row] = L;
}

}  // namespace

hipError_t launch_lse_merge(int heads, int64_t n_q, int dim, int n_parts, const float* const* outs,
                            const float* const* lses, float* out, float* lse, hipStream_t st) {
  const int64_t rows = int64_t(heads) * n_q;
  if (rows == 0) return hipSuccess;
  const int dim4 = dim / 4;
  const int64_t blocks = (rows * dim4 + 255) / 256;
  // Merge in chunks: the first launch merges up to kMaxMergeParts parts into
  // (out, lse); each following launch merges (out, lse) with the next parts.
  int done = 0;
  while (done < n_parts) {
    PartPtrs pp{};
    int k = 0;
    if (done > 0) { pp.o[0] = out; pp.l[0] = lse; k = 1; }
    while (k < kMaxMergeParts && done < n_parts) { pp.o[k] = outs[done]; pp.l[k] = lses[done]; ++k; ++done; }
    hipLaunchKernelGGL(lse_merge_kernel, dim3(unsigned(blocks)), dim3(256), 0, st, pp, k, rows, dim4, out, lse);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_lse_merge_strided(int heads, int64_t n_q, int dim, int n_parts, const float* outs,
                                    const float* lses, float* out, float* lse, hipStream_t st) {
  const float* po[kMaxMergeParts * 4];
  const float* pl[kMaxMergeParts * 4];
  if (n_parts > kMaxMergeParts * 4) return hipErrorInvalidValue;
  const int64_t rows = int64_t(heads) * n_q;
  for (int p = 0; p < n_parts; ++p) { po[p] = outs + p * rows * dim; pl[p] = lses + p * rows; }
  return launch_lse_merge(heads, n_q, dim, n_parts, po, pl, out, lse, st);
}

}  // namespace kvc
