// Launch descriptors of the Lion kernel.
#pragma once
#include "common.hpp"

namespace ma {

constexpr int kMaxLionSegs = 24;
constexpr int kLionBlockElems = 4096;

struct LionSeg {
  float* p;
  const float* g;
  float* m;
  int64_t n;
  int64_t block_begin;
  float lr, cd, b1, b2, c1, c2;
  int32_t decay;
  int32_t vec;   // all three pointers 16-byte aligned
};

struct LionArgs {
  int32_t nseg;
  int32_t total_blocks;
  LionSeg s[kMaxLionSegs];
};

hipError_t launch_lion(const LionArgs& a, hipStream_t s);

}  // namespace ma
