/*
 * fp4idx_ceiling.h -- measurement entry points of libfp4idx: plain HBM
 * traffic of the shapes the producer and the scorer move, with none of the
 * method's arithmetic, so their measured rates can be set against what the
 * same traffic reaches on this GPU; and the VALU issue rate of single
 * instruction kinds, for the kernels bound by vector ALU issue.  Not part of the method; used by the
 * benchmark.  Conventions as in fp4idx.h: device pointers, `stream` a
 * hipStream_t as void* (NULL = default stream), nothing allocated, no
 * synchronization.  Returns 0 on success, 1 for an invalid argument (nothing
 * enqueued), 3 for a HIP error.
 */
#ifndef FP4IDX_CEILING_H
#define FP4IDX_CEILING_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Reads read_bytes from src and writes write_bytes to dst (both multiples of
 * 1,024, both buffers 16-byte aligned) in 1 KB units, the write units spread
 * evenly over the read units while write_bytes <= read_bytes: write_bytes = 0
 * is a read-only stream, equal sizes a copy.  A read-only stream takes four
 * units per wavefront step on two workgroups per compute unit, a stream with
 * writes one unit per step at full occupancy (the shapes that measured
 * fastest for each).  dst receives data derived from src (its contents are of
 * no use) and must hold at least 1,024 bytes even for a read-only stream.
 * Each size is at most 2^40 bytes.  One persistent grid of 16-byte accesses.
 */
int fp4idx_ceiling_stream(const void* src, int64_t read_bytes, void* dst, int64_t write_bytes,
                          void* stream);

/*
 * The access pattern of fp4idx_paged_mqa_logits in decode: for every key block
 * of every sequence (block_table [B, max_blocks] int32, context_lens [B] int32,
 * clamped as the scorer clamps them), reads the block's 4,096 code bytes of
 * kv_cache [NB,1,4,64,16] and its 256-byte row of kv_cache_scale [NB,1,4,64],
 * and writes next_n fp32 values per key into logits [B*next_n, stride] (values
 * of no use), with the scorer's flat, balanced split of the blocks over
 * wavefronts and LDS-DMA loads into a per-wavefront ring.  B <= 1024,
 * next_n <= 64, B * max_blocks < 2^31.
 */
int fp4idx_ceiling_paged_gather(const uint8_t* kv_cache, const uint8_t* kv_cache_scale, int64_t NB,
                                const int32_t* block_table, int64_t max_blocks,
                                const int32_t* context_lens, int64_t B, int next_n, float* logits,
                                int64_t stride, void* stream);

/*
 * VALU issue rate: `workgroups` workgroups of 256 threads, every lane running
 * 8 independent chains of `iterations` steps of one instruction kind, so that
 * with several wavefronts per SIMD the rate at which the SIMDs issue that
 * instruction bounds the launch:
 *   kind 0  fp32 add (v_add_f32), 1  fp32 fused multiply-add with distinct
 *   operands (v_fma_f32), 2  fp32 max (v_max_f32), 3  fp32 pair -> packed
 *   bf16 (v_cvt_pk_bf16_f32), 4  bf16 pair -> E2M1 with a power-of-two scale
 *   (v_cvt_scalef32_pk_fp4_bf16).
 * Lane operations performed: workgroups * 256 * iterations * 8.  out (4-byte
 * aligned) receives workgroups * 256 dwords, one per thread, derived from its
 * chains (values of no use).  kind outside 0..4, workgroups outside
 * [1, 2^20], iterations outside [0, 2^32] or a null out: 1, nothing enqueued.
 */
int fp4idx_ceiling_valu(int kind, int64_t workgroups, int64_t iterations, uint32_t* out,
                        void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FP4IDX_CEILING_H */
