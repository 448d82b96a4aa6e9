/*
 * kvc_probe.h - roofline probes of libkvc.so.
 *
 * Measured denominators for the attention kernels' rooflines, reported beside
 * MI355X's published peaks (dense bf16 matrix cores 2.5 PFLOP/s, HBM3E
 * 8 TB/s).  The attention step is a dense contraction for chunked and global
 * attention, bounded by the matrix cores, and close to the HBM bound for a
 * single frame's queries ("vLLM-Omni RFC #2727: Reconstruction Engine",
 * section 2.2: global attention is the compute and memory bottleneck;
 * "LingBot-Map Paged KV Cache", section 1: each new frame attends to all
 * cached KV).  Each probe runs an untimed launch, then times five launches
 * with HIP events on `stream`, and blocks until they are done.  The caller
 * owns every buffer.  Errors as in kvc.h.
 */
#ifndef KVC_PROBE_H_
#define KVC_PROBE_H_

#include <stddef.h>
#include <stdint.h>

#include "kvc.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes of the device scratch buffer each probe writes its results into. */
size_t kvc_probe_scratch_bytes(void);

/* Dense bf16 matrix-core rate: one workgroup of sixteen waves (four per SIMD)
 * per compute unit, each wave issuing four independent chains of
 * v_mfma_f32_32x32x16_bf16 from registers (32*32*16*2 FLOP each).  *tflops receives the rate in TFLOP/s.
 * scratch: device buffer of kvc_probe_scratch_bytes. */
int kvc_probe_mfma_bf16(void* scratch, size_t scratch_bytes, kvc_stream_t stream, double* tflops);

/* The 512-row attention kernel's per-tile instruction mix on its own: per
 * wave and 64-key tile, the K and V fragment reads from LDS, one workgroup
 * barrier, 32 products (v_mfma_f32_32x32x16_bf16) and the online softmax of two
 * 32-row blocks issued as the kernel issues them (each block's exponentials,
 * FMAs and adds in fenced groups beside the other block's products), with no
 * global memory, table walk, masks or rare-path checks; eight waves and
 * 96 KiB of LDS per workgroup, one workgroup per compute unit.  *tflops
 * receives the products' rate in TFLOP/s: the ceiling that this mix of
 * matrix and vector work sets for the kernel on this chip ("vLLM-Omni RFC
 * #2727: Reconstruction Engine", section 2.2: global attention is the compute
 * bottleneck).  scratch: device buffer of kvc_probe_scratch_bytes. */
int kvc_probe_tile_mix(void* scratch, size_t scratch_bytes, kvc_stream_t stream, double* tflops);

/* HBM bandwidth: a streaming read of `bytes` from src (16-byte loads folded
 * into one word per thread) and a streaming copy of `bytes` from src to dst.
 * *read_gbs receives bytes / time, *copy_gbs (read + written bytes) / time,
 * both in GB/s (1e9 bytes).  src and dst: device buffers of `bytes`, a
 * multiple of 16, 16-byte aligned, much larger than the caches (1 GiB or
 * more) for an HBM figure.  scratch: device buffer of kvc_probe_scratch_bytes. */
int kvc_probe_hbm(const void* src, void* dst, size_t bytes, void* scratch, size_t scratch_bytes,
                  kvc_stream_t stream, double* read_gbs, double* copy_gbs);

#ifdef __cplusplus
}
#endif

#endif /* KVC_PROBE_H_ */
