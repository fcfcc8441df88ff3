/* A plain C99 program that runs one decode step through the C ABI alone
 * (no Python, no torch in the process): it reads the pools, the step's new
 * tokens, the queries and the tables from a binary file, copies them to the
 * GPU with the HIP runtime, calls paged_kv_write then paged_attn_decode, and
 * writes the float32 output. tests/test_gpu_c_abi.py builds the inputs and
 * checks the output against the oracle.
 *
 * Input file: int32 header {num_blocks, block_size, num_heads, num_kv_heads,
 * head_dim, kv_dtype, num_seqs, max_blocks_per_seq, max_context_len,
 * num_tokens}, float32 scale, then k_pool, v_pool [NB, B, Hkv, D] and q
 * [S, H, D] (16-bit), k_new, v_new [T, Hkv, D] (16-bit), seq_idx, pos [T],
 * block_tables [S, MB] and context_lens [S] (int32). */
#include <stdio.h>
#include <stdlib.h>
#include <hip/hip_runtime_api.h>
#include "paged_attn.h"

static void* read_dev(FILE* f, size_t n) {
  void* h = malloc(n ? n : 1);
  void* d = NULL;
  if (!h || fread(h, 1, n, f) != n) { fprintf(stderr, "short input\n"); exit(2); }
  if (hipMalloc(&d, n ? n : 1) != hipSuccess || hipMemcpy(d, h, n, hipMemcpyHostToDevice) != hipSuccess) {
    fprintf(stderr, "hip copy failed\n");
    exit(2);
  }
  free(h);
  return d;
}

int main(int argc, char** argv) {
  if (argc != 3) { fprintf(stderr, "usage: %s in.bin out.bin\n", argv[0]); return 2; }
  FILE* f = fopen(argv[1], "rb");
  if (!f) return 2;
  int32_t hd[10];
  float scale;
  if (fread(hd, 4, 10, f) != 10 || fread(&scale, 4, 1, f) != 1) return 2;
  pkv_geometry_t g = {hd[0], hd[1], hd[2], hd[3], hd[4], hd[5]};
  const int S = hd[6], MB = hd[7], max_len = hd[8], T = hd[9];
  const size_t pool = (size_t)g.num_blocks * g.block_size * g.num_kv_heads * g.head_dim * 2;
  void* k_pool = read_dev(f, pool);
  void* v_pool = read_dev(f, pool);
  void* q = read_dev(f, (size_t)S * g.num_heads * g.head_dim * 2);
  void* k_new = read_dev(f, (size_t)T * g.num_kv_heads * g.head_dim * 2);
  void* v_new = read_dev(f, (size_t)T * g.num_kv_heads * g.head_dim * 2);
  int32_t* seq_idx = (int32_t*)read_dev(f, (size_t)T * 4);
  int32_t* pos = (int32_t*)read_dev(f, (size_t)T * 4);
  int32_t* tables = (int32_t*)read_dev(f, (size_t)S * MB * 4);
  int32_t* lens = (int32_t*)read_dev(f, (size_t)S * 4);
  fclose(f);

  int st = paged_kv_write(&g, k_pool, v_pool, k_new, v_new, seq_idx, pos, T, tables, S, MB, NULL);
  if (st) { fprintf(stderr, "paged_kv_write: %s\n", pkv_status_string(st)); return 1; }
  const size_t ws_bytes = paged_attn_decode_workspace_bytes(&g, S, max_len, 0, 0, 0);
  void* ws = NULL;
  const size_t out_bytes = (size_t)S * g.num_heads * g.head_dim * 4;
  float* out = NULL;
  if (hipMalloc(&ws, ws_bytes) != hipSuccess || hipMalloc((void**)&out, out_bytes) != hipSuccess) return 2;
  st = paged_attn_decode(&g, out, NULL, q, k_pool, v_pool, tables, MB, lens, S, max_len, 0, 0, scale, 0, ws,
                         ws_bytes, NULL);
  if (st) { fprintf(stderr, "paged_attn_decode: %s\n", pkv_status_string(st)); return 1; }
  float* host = (float*)malloc(out_bytes);
  if (!host || hipMemcpy(host, out, out_bytes, hipMemcpyDeviceToHost) != hipSuccess) return 2;
  FILE* o = fopen(argv[2], "wb");
  if (!o || fwrite(host, 1, out_bytes, o) != out_bytes) return 2;
  fclose(o);
  printf("c abi decode ok: %d sequences, %zu workspace bytes\n", S, ws_bytes);
  return 0;
}
