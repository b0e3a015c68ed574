// Internal helpers shared by the library's translation units (not part of the ABI).
#pragma once
#include <cstdarg>
#include <cstdint>

#include "kvq.h"

namespace kvq {

constexpr int kHeadDim = 128;
constexpr int kPage = 16;
constexpr int kGroup = 32;
constexpr int kMaxG = 16;             // query heads per KV head handled by the decode kernel
constexpr int kMaxReorderEntries = 32768;  // entries per table the reorder stages in LDS (4 B each)

// Head block sizes and region offsets (the written layout; see kvq.h).  Code rows are
// little-endian 32-bit words; with b bits per code, word w holds channels
// w*32/b .. (w+1)*32/b - 1, even-indexed ones in the low 16 bits and odd-indexed ones
// in the high 16 bits, ascending, b bits each.  INT4 K meta is token-major
// [16][4 groups][s, z]; INT4 V meta is group-major [4][16][s, z]; INT2 V meta is, per
// group (64 B), the 16 tokens' fp16 scales, then their 16 fp16 zeros; INT2 K meta is 64
// fp16 scales then 64 fp16 zeros per page (even page: channels 0-63).
constexpr int kI4Bytes = 2560, kI4KC = 0, kI4KM = 1024, kI4VC = 1280, kI4VM = 2304;
constexpr int kI2Bytes = 1536, kI2KC = 0, kI2KS = 512, kI2KZ = 640, kI2VC = 768, kI2VM = 1280;
constexpr int kF16Bytes = 8192, kF16K = 0, kF16V = 4096;
// FP8 anchor block (the FP16 class of a cache with FP8 anchors): e4m3 codes and one
// power-of-two fp16 scale per token, K then V.
constexpr int kF8Bytes = 4160, kF8K = 0, kF8KS = 2048, kF8V = 2080, kF8VS = 4128;

// Records a formatted message as this thread's last error and returns `st`.
kvq_status fail(kvq_status st, const char *fmt, ...);

// Validates the host-visible fields of a cache descriptor.
kvq_status check_cache(const kvq_cache *c);

}  // namespace kvq
