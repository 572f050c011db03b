// Launch descriptors of the AdamW kernel.
#pragma once
#include "common.hpp"

namespace ma {

constexpr int kMaxAdamSegs = 24;
constexpr int kAdamBlockElems = 4096;

struct AdamSeg {
  float* p;
  const float* g;
  float* m;
  float* v;
  int64_t n;
  int64_t block_begin;
  float cd, b1, b2, c1, c2, ss, s2, eps;
  int32_t decay;
  int32_t vec;   // all four pointers 16-byte aligned
};

struct AdamArgs {
  int32_t nseg;
  int32_t total_blocks;
  int32_t lean_blocks;   // > 0: k_adamw_lean with this many workgroups (at most)
  AdamSeg s[kMaxAdamSegs];
};

hipError_t launch_adamw(const AdamArgs& a, hipStream_t s);

}  // namespace ma
