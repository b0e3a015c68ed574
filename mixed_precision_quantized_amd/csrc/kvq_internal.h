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
constexpr int kMaxReorderEntries = 8192;

// Head block sizes and region offsets (the written layout; see kvq.h).
constexpr int kI4Bytes = 2560, kI4KC = 0, kI4KM = 1024, kI4VC = 1280, kI4VM = 2304;
constexpr int kI2Bytes = 1536, kI2KC = 0, kI2KM = 512, kI2VC = 768, kI2VM = 1280;
constexpr int kF16Bytes = 8192, kF16K = 0, kF16V = 4096;

// Records a formatted message as this thread's last error and returns `st`.
kvq_status fail(kvq_status st, const char *fmt, ...);

// Validates the host-visible fields of a cache descriptor.
kvq_status check_cache(const kvq_cache *c);

}  // namespace kvq
