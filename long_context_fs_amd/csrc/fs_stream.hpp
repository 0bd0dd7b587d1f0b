// fs_stream.hpp -- layout of the streaming FS-L state (host and device view).
//
// FreeSolo summary, "Bounded memory" under Practical Implications: FS-L's
// streaming cache keeps O((P + W) s + w + B + s) d token state per head,
// whatever the sequence length.  Per (batch, head) the state holds
//  * a mirrored ring of the last L token keys and values, L a power of two
//    >= w + s + B (B = most tokens per step): token p sits at rows p mod L and
//    p mod L + L, so any L consecutive positions are contiguous;
//  * a pool of M = W + P + ceil(B / s) + 2 cell slots with the retained cells'
//    raw keys and values (s rows each), kbar, a_c and cell index (eq. 5);
//  * eq. 8's TopP set as (a_c, c, slot) entries in ascending c, the slots of the
//    W most recent candidate cells, a free-slot list and the slots to free at
//    the next step;
//  * the keep rows (slot lists, ascending cell) of the step's candidate counts.
// Step-sized scratch (selected slots, the two branch outputs, the RoPE table,
// the readout's split workspace) follows the per-head arrays.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace fs {

struct StreamCfg {
    int B, H, d, s, w, W, P, K, max_new;
    int bf16;
    double rope_base;
    float rms_eps;
};

struct StreamLayout {
    int L;        // ring rows per copy
    int M;        // pool slots
    int R;        // keep rows per step
    int keep_w;   // W + P
    int esize;    // bytes per stored element
    // byte offsets of [B*H][...] arrays, then of the step scratch
    size_t hdr, ring_k, ring_v, pool_k, pool_v, kbar, amax, cell, topp_a, topp_c, topp_s, recent,
        free_list, pend, keep, keep_cnt;
    size_t idx, osr, olr, table, table_bytes, ws, ws_bytes, bytes;
};

// Header words per (batch, head).
enum StreamHdr {
    kHdrTokens = 0,    // tokens appended since reset
    kHdrCells = 1,     // candidate cells processed (n of the last query)
    kHdrTopP = 2,      // entries in TopP
    kHdrFree = 3,      // free slots
    kHdrPend = 4,      // slots to free at the next step
    kHdrError = 5,     // nonzero: a step found no free slot (cannot happen within the sizes above)
    kHdrWords = 16
};

StreamLayout stream_layout(const StreamCfg& c);

}  // namespace fs
