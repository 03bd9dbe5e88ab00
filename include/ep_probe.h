/*
 * ep_probe.h -- C ABI of libep_probe.so: streaming HBM probes that measure
 * the bandwidth a kernel can reach on this GPU for plain reads, writes and
 * copies.  They give the achievable ceilings the shuffle's kernels are
 * compared against (next to the published 8 TB/s peak): dispatch is bound
 * by HBM writes, combine by HBM reads.  Not part of the shuffle itself.
 *
 * The shuffle's own measurement on the pages is bandwidth in GB/s per
 * stage ("DeepEP V1 vs V2 深度对比分析" §4.3); these probes fix what GB/s one
 * MI355X can deliver to a single kernel.
 */
#ifndef EP_AMD_EP_PROBE_H
#define EP_AMD_EP_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { EP_PROBE_READ = 0, EP_PROBE_WRITE = 1, EP_PROBE_COPY = 2 };

/* One launch of a streaming kernel over `bytes` (a multiple of 16 *
 * threads * vec_per_lane) of device memory, on `stream` (a hipStream_t):
 *   EP_PROBE_READ: reads d_src; writes at most one 16-byte word per
 *     workgroup into d_dst (which needs blocks * 16 bytes) so the loads
 *     cannot be dropped;
 *   EP_PROBE_WRITE: writes d_dst (its previous contents are overwritten);
 *   EP_PROBE_COPY: copies d_src to d_dst.
 * blocks workgroups of threads threads (64..1024, a multiple of 64) walk the
 * buffer in a grid-stride loop, each thread moving vec_per_lane (1, 2, 4 or
 * 8) 16-byte vectors per step, lane-contiguous; nontemporal != 0 gives the
 * loads and stores the non-temporal hint.  Returns 0, or -1 for invalid
 * arguments, or the HIP error code of the launch. */
int ep_probe_stream(int mode, const void* d_src, void* d_dst, int64_t bytes, int blocks,
                    int threads, int vec_per_lane, int nontemporal, void* stream);

/* The shuffle's two row access patterns without their arithmetic, one wave
 * per (token, chunk of 64 * vec_per_lane 16-byte vectors), as the kernels
 * do them, for the patterns' own ceilings:
 *   EP_PROBE_GATHER (the combine's): for each token t < num_tokens, row t of
 *     d_dst = XOR over k < topk with d_slot[t*topk + k] >= 0 of row
 *     d_slot[t*topk + k] of d_src; all of a chunk's loads are issued first;
 *   EP_PROBE_SCATTER (the dispatch's): for each token t and k with a slot,
 *     row d_slot[t*topk + k] of d_dst = row t of d_src.
 * Rows are row_bytes long (a multiple of 16); d_slot int32 [num_tokens,
 * topk] with entries < the rows of the indexed buffer (the caller's
 * guarantee); topk 1..16; threads 64..1024, a multiple of 64;
 * vec_per_lane 1, 2 or 4; non-temporal loads and stores.  Returns 0, -1 for
 * invalid arguments, or the HIP error code of the launch. */
enum { EP_PROBE_GATHER = 3, EP_PROBE_SCATTER = 4 };
int ep_probe_rows(int mode, const void* d_src, void* d_dst, const int32_t* d_slot,
                  int64_t num_tokens, int topk, int64_t row_bytes, int threads, int vec_per_lane,
                  void* stream);

#ifdef __cplusplus
}
#endif

#endif
