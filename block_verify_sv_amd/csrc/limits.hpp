// Size limits shared by the libspecverify kernels and their host checks.
#pragma once

namespace sv {

constexpr int kNumCUs = 256;      // MI355X compute units (8 XCDs x 32)
constexpr int kMaxBlock = 64;     // K limit (one uint64 mask row per block row)
constexpr int kMaxRows = 512;     // K * G limit of one KV head (2 row groups of 256, 4 of 128 for fp32)
constexpr int kMaxSplitKeys = 16384;  // keys of one split-KV work item

}  // namespace sv
