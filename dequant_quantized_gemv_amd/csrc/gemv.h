// gemv.h - launch descriptors of the fused quantized GEMV (host and device).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qk {

constexpr int kGvChunkPairs = 64;                   // pairs per 4096-weight chunk
constexpr int kGvChunkElems = kGvChunkPairs * 64;   // weights per activation window

// One problem of a (possibly grouped) launch: y = W x for NC columns.
struct GemvItem {
    const uint8_t *w;
    const float *x;
    float *y;
    int64_t ldx;
    int64_t ldy;
    int m;
    int nb;  // blocks per row
};

constexpr int kGvMaxItems = 16;

// A table of up to kGvMaxItems problems (passed by value in the kernel
// argument segment).  Row groups of all items are numbered consecutively:
// item i owns groups gbase[i] .. gbase[i+1]-1 (filled in by the launcher).
struct GemvArgs {
    GemvItem item[kGvMaxItems];
    int gbase[kGvMaxItems + 1];
    int sub[kGvMaxItems];  // per-problem lane split of a one-column launch whose problems differ in it
    int count;
};

// Expert-indexed problems (one column each): for token t and slot s,
// item t*n_used + s multiplies expert ids[t*ld_ids + s] of the stack at w
// (experts estride bytes apart) by x + t*x_tok + s*x_slot into
// y + t*y_tok + s*y_slot.  The id is read on the device.
struct GemvExpert {
    const uint8_t *w;
    int64_t estride;
    const int32_t *ids;
    int64_t ld_ids;
    const float *x;
    int64_t x_slot;
    int64_t x_tok;
    float *y;
    int64_t y_slot;
    int64_t y_tok;
    int m;
    int nb;      // blocks per row
    int nexp;    // experts in the stack
    int n_used;  // slots per token
    int count;   // tokens * slots
};

// Launch one table of problems with NC columns each (count == 1 uses the
// single-problem kernel).  `fast`: every w 4-byte aligned with an even number
// of blocks per row.
template <int NC>
int gemv_table(int fmt, GemvArgs &a, bool fast, hipStream_t stream);

// The same with 8-bit activations (integer dot products); one problem only.
template <int NC>
int gemv_table_x8(int fmt, GemvArgs &a, bool fast, hipStream_t stream);

// Launch expert-indexed problems (same `fast` condition, for every expert and
// slot).
int gemv_expert(int fmt, const GemvExpert &e, bool fast, hipStream_t stream);

}  // namespace qk
