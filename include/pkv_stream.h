/* Streaming-read reference kernel (libpkvstream.so).
 *
 * Not part of the attention path: a plain contiguous read of a device buffer
 * that the benchmark times beside the decode, so that the decode's bandwidth
 * can be read against what a simple stream achieves on the same GPU, not
 * only against the published HBM peak.  Decode attention is bound by the
 * bandwidth of reading the KV history ("从正确到更快：PagedAttention 的优化
 * 路线", section "先明确优化目标：我们到底在优化什么"; "算子与编译器：推理
 * Attention 与 KV Kernel", section "2. Prefill Attention 与 Decode Attention
 * 的差异"), so a plain stream read is its natural yardstick.
 */
#ifndef PKV_STREAM_H
#define PKV_STREAM_H

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Enqueue one read of `bytes` bytes at device address `src` on `stream`.
 *  src    device pointer, 16-byte aligned, owned by the caller; only read.
 *  bytes  > 0 and a multiple of 16.
 *  sink   device pointer to one uint32_t owned by the caller; written only
 *         when the folded data hash equals a fixed constant (it exists so
 *         that the loads cannot be optimised away).
 * Returns 0 when the launch was enqueued, -1 for a null pointer, a
 * misaligned pointer or a bad size (nothing is launched), otherwise the
 * hipError_t of the launch. */
int pkv_stream_read(const void *src, int64_t bytes, uint32_t *sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif
