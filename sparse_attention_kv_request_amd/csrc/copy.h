// Miss copy (copy.hip): its arguments and launch shape.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace hisparse {

// Launch shape of the miss copy; the macros let a build sweep other shapes.
#ifndef HISPARSE_COPY_THREADS
#define HISPARSE_COPY_THREADS 256
#endif
#ifndef HISPARSE_COPY_UNROLL
#define HISPARSE_COPY_UNROLL 4
#endif
#ifndef HISPARSE_COPY_BLOCKS
#define HISPARSE_COPY_BLOCKS 1024
#endif
#ifndef HISPARSE_COPY_ROW_BLOCKS
#define HISPARSE_COPY_ROW_BLOCKS 256
#endif
#ifndef HISPARSE_FUSE_MIN_ROWS
#define HISPARSE_FUSE_MIN_ROWS 16
#endif
#ifndef HISPARSE_COPY_NT_LOAD
#define HISPARSE_COPY_NT_LOAD 0
#endif

constexpr int kCopyThreads = HISPARSE_COPY_THREADS;
constexpr int kCopyUnroll = HISPARSE_COPY_UNROLL;  // 16-byte loads in flight per lane
// Workgroups: 4 per CU on 256 CUs for whole pages (units of 4 KiB and more),
// one per CU for token rows.  Measured on the 64-request swap step (656-B
// rows, alternated three times on one box): 256 workgroups copy a launch in
// 333.6 us against 335.3 us with 1024 (128 took 351 us, 64 varied from 332
// to 335 us); with 168-KB pages 1024 stay 0.2 % ahead.
constexpr int kCopyBlocks = HISPARSE_COPY_BLOCKS;
constexpr int kCopyRowBlocks = HISPARSE_COPY_ROW_BLOCKS;
constexpr int64_t kCopyPageUnit = 4096;
// Token-row swap calls of at least this many rows copy inside the plan
// kernel: each row's workgroup moves its own misses (8 loads in flight per
// lane) once its commit is done, so the copy starts without a second launch.
// Measured per step against the separate copy kernel: 64 rows x 8 layers
// 2.681 vs 2.741 ms, 32 rows 1.403 vs 1.441, 16 rows 0.776 vs 0.785, 8 rows
// even, one row 3x slower (one workgroup keeps too few host reads in
// flight); 168-KB pages 4 % slower (the copy kernel spreads a row's pages
// over many workgroups), so page mode always uses it.  The plan kernel's
// entries are in range by construction; the copy kernel checks each one
// because a replayed plan comes from the caller.
constexpr int kFuseMinRows = HISPARSE_FUSE_MIN_ROWS;

// Rows of `unit_bytes` from the host tier to the hot buffer.
struct CopyArgs {
  const int32_t* miss_count;  // [batch]
  const int32_t* src;         // [batch][cap] host row
  const int32_t* dst;         // [batch][cap] device row
  int32_t batch;
  int32_t cap;
  const uint8_t* host;        // device-visible address of the host tier
  uint8_t* dev;
  int32_t unit16;             // 16-byte chunks per row
  int64_t unit_bytes;
  int64_t src_rows;           // valid host rows [0, src_rows)
  int64_t dst_rows;           // valid device rows [0, dst_rows)
  uint32_t* err;
};

hipError_t launch_miss_copy(const CopyArgs& a, hipStream_t s);

}  // namespace hisparse
