// Hard tile-configuration sample: per-tile dense / 2:4 choice and per-group
// 2:4 pattern from logits plus Gumbel noise, written as a bit-packed keep
// mask that patch_pack accepts.
//
// PATCH learns a per-tile choice between dense and 2:4 ("PATCH: Learnable
// Tile-level Hybrid Sparsity for LLMs", Abstract) from logits sampled with
// Gumbel noise under a scaling kappa (model card "llama_3.2_1b-PATCH-45Sparse",
// "Training hyper-parameters"), and the pattern inside a 2:4 group from
// logits over its candidate patterns (card "gemma_3_1b-MaskLLM-50Sparse",
// description).  A hard sample takes, per choice, the index of the largest
// fl(fl(kappa * logit) + noise) in fp32; the first maximum wins and a NaN
// score never wins.  The temperature divides all scores of a choice by the
// same positive number, so it does not enter a hard sample.
#include "patch_internal.h"

namespace {

// Keep bits (bit j = position j of the group) of the six 2:4 patterns, in the
// order (0,1) (0,2) (0,3) (1,2) (1,3) (2,3).
__constant__ uint8_t kPatternKeep[6] = {0x3, 0x5, 0x9, 0x6, 0xA, 0xC};

__device__ __forceinline__ float score(float kappa, float logit, float noise) {
#pragma clang fp contract(off)
  const float p = kappa * logit;  // rounded on its own: no fused multiply-add
  return p + noise;
}

template <int C>
__device__ __forceinline__ int first_max(const float* logit, const float* noise, float kappa) {
  float best = -__builtin_inff();
  int idx = 0;
#pragma unroll
  for (int i = 0; i < C; ++i) {
    const float s = score(kappa, logit[i], noise ? noise[i] : 0.0f);
    if (s > best) {  // ties keep the lower index; NaN never compares greater
      best = s;
      idx = i;
    }
  }
  return idx;
}

// One thread per mask byte: 8 consecutive k of one row, i.e. two groups.
__global__ void k_sample_mask(const float* __restrict__ tile_logits, const float* __restrict__ tile_noise,
                              const float* __restrict__ group_logits, const float* __restrict__ group_noise,
                              int64_t n, int64_t k, int tn, int tk, int64_t tiles_k, float kappa, int lsb_first,
                              uint8_t* __restrict__ bits) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row_bytes = k / 8;
  if (i >= n * row_bytes) return;
  const int64_t row = i / row_bytes, c8 = i % row_bytes;
  const int64_t t = (row / tn) * tiles_k + (c8 * 8) / tk;
  const bool dense =
      first_max<2>(tile_logits + 2 * t, tile_noise ? tile_noise + 2 * t : nullptr, kappa) == 0;
  uint32_t keep = 0xFF;  // bit j = k offset j of the byte's 8 weights
  if (!dense) {
    const int64_t g0 = row * (k / 4) + 2 * c8;  // first of the byte's two groups
    keep = 0;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t off = (g0 + h) * 6;
      const int p = first_max<6>(group_logits + off, group_noise ? group_noise + off : nullptr, kappa);
      keep |= (uint32_t)kPatternKeep[p] << (4 * h);
    }
  }
  // MSB first: weight j of the byte is bit 7 - j
  bits[i] = (uint8_t)(lsb_first ? keep : (__builtin_bitreverse32(keep) >> 24));
}

}  // namespace

hipError_t launch_sample_mask(const float* tile_logits, const float* tile_noise, const float* group_logits,
                              const float* group_noise, int64_t n, int64_t k, int tn, int tk, float kappa,
                              int lsb_first, uint8_t* bits, hipStream_t s) {
  const int64_t bytes = n * k / 8;
  if (bytes == 0) return hipSuccess;
  const int threads = 256;
  const int64_t blocks = (bytes + threads - 1) / threads;
  hipLaunchKernelGGL(k_sample_mask, dim3((unsigned)blocks), dim3(threads), 0, s, tile_logits, tile_noise,
                     group_logits, group_noise, n, k, tn, tk, k / tk, kappa, lsb_first, bits);
  return hipGetLastError();
}
