// Status strings, ABI version, per-thread error detail and the document-index
// helpers (chunk CSR and the inverse chunk -> document map).
#include "common.h"

namespace msa {

static thread_local std::string g_last_error;

void set_error(const std::string& msg) { g_last_error = msg; }

int fail(int status, const std::string& msg) {
  g_last_error = msg;
  return status;
}

// chunk_doc[c] = document owning chunk c.  One thread per document writes
// its own chunk range (documents are disjoint ranges of the chunk CSR).
__global__ void chunk_doc_kernel(const int64_t* __restrict__ chunk_off, int64_t n_docs, int64_t n_chunks,
                                 int32_t* __restrict__ chunk_doc) {
  int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n_docs) return;
  int64_t lo = chunk_off[i], hi = chunk_off[i + 1];
  if (lo < 0) lo = 0;
  if (hi > n_chunks) hi = n_chunks;
  for (int64_t c = lo; c < hi; ++c) chunk_doc[c] = int32_t(i);
}

}  // namespace msa

extern "C" {

int msa_abi_version(void) { return 14; }

const char* msa_status_string(int status) {
  switch (status) {
    case MSA_OK: return "ok";
    case MSA_ERR_INVALID_ARG: return "invalid argument";
    case MSA_ERR_UNSUPPORTED: return "unsupported configuration";
    case MSA_ERR_WORKSPACE: return "workspace too small";
    case MSA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* msa_last_error(void) { return msa::g_last_error.c_str(); }

int msa_chunk_offsets(const int64_t* tok_off_h, int64_t n_docs, int chunk, int64_t* chunk_off_h) {
  MSA_REQUIRE(tok_off_h && chunk_off_h, MSA_ERR_INVALID_ARG, "msa_chunk_offsets: NULL pointer");
  MSA_REQUIRE(n_docs >= 1, MSA_ERR_INVALID_ARG, "msa_chunk_offsets: n_docs < 1");
  MSA_REQUIRE(chunk >= 1, MSA_ERR_INVALID_ARG, "msa_chunk_offsets: chunk < 1");
  MSA_REQUIRE(tok_off_h[0] == 0, MSA_ERR_INVALID_ARG, "msa_chunk_offsets: tok_off[0] != 0");
  for (int64_t i = 0; i < n_docs; ++i)
    MSA_REQUIRE(tok_off_h[i + 1] >= tok_off_h[i], MSA_ERR_INVALID_ARG,
                "msa_chunk_offsets: tok_off decreases at document " + std::to_string(i));
  chunk_off_h[0] = 0;
  for (int64_t i = 0; i < n_docs; ++i) {
    int64_t len = tok_off_h[i + 1] - tok_off_h[i];
    chunk_off_h[i + 1] = chunk_off_h[i] + (len + chunk - 1) / chunk;
  }
  msa::set_error("");
  return MSA_OK;
}

int msa_chunk_doc_map(const int64_t* chunk_off, int64_t n_docs, int64_t n_chunks, int32_t* chunk_doc,
                      void* stream) {
  MSA_REQUIRE(chunk_off && chunk_doc, MSA_ERR_INVALID_ARG, "msa_chunk_doc_map: NULL pointer");
  MSA_REQUIRE(n_docs >= 1 && n_chunks >= 1, MSA_ERR_INVALID_ARG, "msa_chunk_doc_map: empty memory");
  MSA_REQUIRE(n_docs < (int64_t(1) << 31), MSA_ERR_UNSUPPORTED, "msa_chunk_doc_map: n_docs >= 2^31");
  const int threads = 256;
  const int64_t blocks = (n_docs + threads - 1) / threads;
  hipLaunchKernelGGL(msa::chunk_doc_kernel, dim3(unsigned(blocks)), dim3(threads), 0, msa::as_stream(stream),
                     chunk_off, n_docs, n_chunks, chunk_doc);
  MSA_LAUNCH_CHECK();
  return MSA_OK;
}

}  // extern "C"
