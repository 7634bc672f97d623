// Host-side launchers of the gfx950 kernels (internal to the library; the
// public C ABI is include/dsa_indexer.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsa {

// Devices the per-device caches of the launchers cover (others query each
// time).
constexpr int kMaxDevices = 64;

struct LogitsArgs {
  const uint8_t* q8;            // e4m3fn codes [T, H, 128]
  const float* q_scale;         // [T, H]
  const float* weights;         // [T, H]
  const uint8_t* k_cache;       // [num_pages, 8448]
  int64_t num_pages;
  const int32_t* block_table;   // [R, bt_stride]
  int64_t bt_stride;
  const int32_t* qsl;           // query_start_loc [R + 1]
  const int32_t* positions;     // [T]
  int64_t T;
  int R;
  int H;
  float* logits;                // [T, ld]
  int64_t ld;
  // 16-row tile kernel only: score logical pages j = 0, 1, .. of the real
  // pages j * page_stride (the fused forward's sample pass) and write row t
  // at logits + t * out_ld (0: ld), page j at columns 64 j ..
  int page_stride = 1;
  int64_t out_ld = 0;
};

// Candidate mode of the 16-row tile kernel (fused forward): instead of its
// logits, workgroup (tile, split x) appends the (ordered key, column) of
// every logit of row t at or above tlo[t] to cand[(t * splits + x) * cap
// ..], in ascending column order, and writes how many there were (possibly
// more than cap) to count[t * splits + x].
struct FusedTile {
  const uint32_t* tlo = nullptr;
  uint2* cand = nullptr;
  uint32_t* count = nullptr;
  int cap = 0;
};

struct TopkArgs {
  const float* logits;          // [T, ld]
  int64_t ld;
  const int32_t* positions;     // [T]
  int64_t T;
  int k;
  int32_t* out;                 // [T, out_ld]
  int64_t out_ld;
  void* workspace;
  size_t ws_bytes;
  // Rows with a position >= pos_limit get a row of -1 (0: ld).  The forward
  // pass sets min(ld, 64 * bt_stride): the logits kernels leave such a row
  // unscored.
  int64_t pos_limit = 0;
};

// One layer's hot path: q quantisation into q8 / q_scale, logits, top-k.
struct ForwardArgs {
  const uint16_t* q_bf16;       // [T, H, 128]
  uint8_t* q8;                  // lg.q8
  float* q_scale;               // lg.q_scale
  LogitsArgs lg;
  TopkArgs tk;                  // tk.logits == lg.logits
  // decode page schedule (logits_schedule_bytes(T, ld) bytes), or null;
  // build_sched false: it already holds the schedule of this batch's
  // positions, query_start_loc and block table (IndexCache F layers)
  int32_t* sched = nullptr;
  bool build_sched = true;
};
// Bytes of the decode page schedule of a T-row batch with ld-column logits
// (0 when no schedule is used for such a batch).
size_t logits_schedule_bytes(int64_t T, int64_t ld);
hipError_t launch_logits_schedule(const LogitsArgs& a, int32_t* sched,
                                  hipStream_t stream);

// Kernel-choice knobs (dsa_set_option); 0 = automatic.  Kept per device as
// atomics; options() is a snapshot of the calling thread's current device.
struct Options {
  int logits_kernel = 0;        // 1 row-wise, 2 tiled 8x2, 3 tiled direct, 4 row grid, 5 tiled 16x1 with the two-op epilogue, 6 tiled 16x1 (the default tiled kernel, forced)
  int row_pages_per_wave = 0;
  int tile_pages_per_split = 0;
  int row_head_waves = 0;       // decode: 1 + head waves per row (0: one)
  int topk_kernel = 0;          // 0/1 register rows, 2 LDS-cached rows, 3 long rows by multi-WG radix, register rows: 0 two 512-thread workgroups per CU when rows outnumber CUs, else one 1024-thread, 1 always 1024, 4 always 512
  int tile_pages_per_step = 0;  // 16-row tile kernel: pages per copy step (0 auto, 2 or 4)
  int fused_sample_stride = 0;  // fused forward: sample every n-th page (0: 32; 16, 32, 64)
  int fused_cand_cap = 0;       // fused forward: candidates per (row, split) slot (0 auto; n: at most n)
  int fused_force_rescue = 0;   // fused forward: 1 re-scores every row of more than k columns
  int fused_select = 0;         // fused forward: candidate select kernel (0 auto, 1/2 one wave per row with 64/80 items per lane (16 splits or fewer), 3 1024-thread workgroup per row)
};
Options options();

hipError_t launch_quantize_q(const uint16_t* q_bf16, int64_t blocks,
                             uint8_t* q8, float* q_scale, hipStream_t stream);
hipError_t launch_forward(const ForwardArgs& f, hipStream_t stream);
hipError_t launch_slot_mapping(const int32_t* block_table, int64_t bt_stride,
                               const int32_t* qsl, int R,
                               const int32_t* positions, int64_t T,
                               int64_t* slots, hipStream_t stream);
hipError_t launch_compressed_slot_mapping(
    const int32_t* block_table, int64_t bt_stride, const int32_t* qsl, int R,
    const int32_t* positions, int64_t T, int ratio, int block_size,
    int64_t* slots, int32_t* positions_c, hipStream_t stream);
hipError_t launch_k_write(const uint16_t* k, int64_t N, const int64_t* slots,
                          uint8_t* k_cache, int64_t num_pages,
                          hipStream_t stream);
hipError_t launch_topk_to_slots(const int32_t* topk, int64_t T, int k,
                                int64_t topk_ld, const int32_t* block_table,
                                int64_t bt_stride, const int32_t* qsl, int R,
                                int64_t* slots, hipStream_t stream);
hipError_t launch_topk_mask(const int32_t* topk, int64_t T, int k,
                            int64_t topk_ld, float* mask, int64_t ld,
                            hipStream_t stream);
// Logits kernel class.  Every class computes each (row, token) logit with
// one fixed sequence of operations, so a row's logits depend on its class
// only, not on which other rows share the launch.
enum class LogitsPlan {
  Auto,      // logits_plan(T, R) of this launch
  Balanced,  // decode: pages dealt out evenly over waves (T <= 128)
  Rowwise,   // one row per workgroup column
  Tiled,     // 16-row tiles of one request through LDS
};
LogitsPlan logits_plan(int64_t T, int R);
int device_cu_count();            // compute units of the current device
hipError_t launch_logits(const LogitsArgs& a, hipStream_t stream,
                         LogitsPlan plan = LogitsPlan::Auto,
                         const int32_t* sched = nullptr);
// The forward pass over row chunks [a, a + rows) that reuse one logits
// buffer: q quantised once, then per chunk query_start_loc rebased into
// qsl_chunk, logits of the chunk's rows (the class of the whole batch) and
// their top-k into rows a.. of the output.
struct ChunkedForwardArgs {
  ForwardArgs f;                // whole batch; f.lg.logits / f.tk.* = chunk
  int64_t rows;                 // rows per chunk (>= 1)
  int32_t* qsl_chunk;           // [R + 1] scratch
};
hipError_t launch_forward_chunked(const ChunkedForwardArgs& c,
                                  hipStream_t stream);
// Fused forward, tile passes (the default tiled class).  Sample pass: the
// logits of every page_stride-th page of each row into samp (row t at samp
// + t * ld_s, logical page j at columns 64 j ..).  Candidate pass: every
// page scored, logits at or above each row's threshold appended to ft
// (FusedTile) over gx page splits per tile -- gx must be
// fused_candidate_splits(a), which the caller sizes ft by.
int64_t fused_candidate_splits(const LogitsArgs& a);
hipError_t launch_logits_sample(const LogitsArgs& a, int page_stride,
                                float* samp, int64_t ld_s, hipStream_t stream);
hipError_t launch_logits_candidates(const LogitsArgs& a, const FusedTile& ft,
                                    int64_t gx, hipStream_t stream);
// The fused forward of a tiled batch: q quantisation into f.q8 / f.q_scale,
// then scoring and exact top-k into f.tk.out without a logits buffer
// (f.lg.logits and f.tk.logits unused); ws holds fused_workspace_bytes(T,
// ld, k) bytes.  The top-k equals launch_forward's with the default tiled
// logits kernel.
size_t fused_workspace_bytes(int64_t T, int64_t ld, int k);
hipError_t launch_forward_fused(const ForwardArgs& f, void* ws,
                                hipStream_t stream);
hipError_t launch_topk(const TopkArgs& a, hipStream_t stream);
size_t topk_workspace_bytes(int64_t T, int64_t ld, int k);
hipError_t read_error_flags(unsigned* flags, bool reset);

}  // namespace dsa
