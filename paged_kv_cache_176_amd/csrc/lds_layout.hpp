// Chunk swizzles of the LDS rings: the 16-byte chunk c of a key's row sits at chunk slot
// c ^ swz(key) (within groups of 8 chunks, or of 4 for 320-byte rows), both when the
// direct global->LDS loads place it and when the operand reads fetch it.  Shared by the
// kernels and, built for the host, by the layout test.
//
// The bank rule they are built for was measured on gfx950 with the LDS bank-conflict
// counter on fixed per-lane address patterns: 64 banks of 4 bytes, and a 64-bit read
// (ds_read_b64, ds_read_b64_tr_b16) served 32 lanes at a time, so a conflict-free 64-bit
// read has each 32-lane half cover the 64 banks once.  128-bit reads follow a rule no
// simple lane grouping reproduces; the swizzles below were measured conflict-free for the
// kernels' 16-byte K-operand reads.
#pragma once
#include <hip/hip_runtime.h>

namespace pa {

// 640- and 1152-byte rows (bf16 DiffKV and MLA): both pitches are 128 bytes mod 256, so
// odd keys sit half a bank space past even ones.  The transposing V^T read puts 8 keys on
// a 32-lane half (4 lanes, 32 bytes = one chunk pair, per key); XOR-ing with key & 6
// gives keys 0, 2, 4, 6 (and 1, 3, 5, 7) four different chunk pairs, so the half covers
// the 64 banks once.  Depends on key bits 1-2 only (any 16-key half of a tile shares it).
__host__ __device__ constexpr int row_chunk_swz(int key) { return key & 6; }

// 320-byte rows (fp8 DiffKV): a pitch of 20 chunks leaves 4 distinct bank offsets per 4
// rows; chunks are permuted within groups of 4, distinct for the 4 keys of one offset
// class and for the 4 keys of one parity in every 8-key half.
__host__ __device__ constexpr int fp8_chunk_swz(int key) { return ((key >> 2) ^ (key >> 1)) & 3; }

// Prefill K rows (384 bytes): a permutation over any 8 consecutive keys, distinct in (key
// parity, swizzle) over 16 keys.  Depends on key bits 0-3 only.
__host__ __device__ constexpr int prefill_k_swz(int key) { return ((key >> 1) ^ (key << 2)) & 7; }

// Prefill V rows (256 bytes: every row spans the 64 banks): the V^T read puts 4 keys x 64
// bytes on a 32-lane half; (key & 3) << 2 gives the 4 keys 4 different 64-byte quarters.
__host__ __device__ constexpr int prefill_v_swz(int key) { return (key & 3) << 2; }

}  // namespace pa
