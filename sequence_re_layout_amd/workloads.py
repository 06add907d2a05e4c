"""Named attention-boundary shapes of the pages' evaluation (Llama and Qwen
models; BASP review page, "Summary" and "Key claims under review").

The pages name the models and the sequence/batch settings but print no head
counts; the counts below are those of the named public model architectures.
Every entry is (name, N, B, S, Hq, Hkv, d); N is the number of (virtual)
ranks, B the micro-batch, S the sequence length, Hq/Hkv the query and
key/value heads, d the head dimension.  Activations are bf16.
"""

TINY = ("tiny", 4, 2, 1024, 8, 8, 64)
LLAMA_1B = ("llama3.2-1b_s16k_b2", 8, 2, 16384, 32, 8, 64)
QWEN_1_8B = ("qwen1.5-1.8b_s16k_b2", 8, 2, 16384, 16, 16, 128)
BATCH_SWEEP = [("llama3.2-1b_s8k_b%d" % B, 8, B, 8192, 32, 8, 64) for B in (1, 2, 4, 8)]
LONG_CONTEXT = [("llama3.2-3b_s%dk_b2" % (S // 1024), 8, 2, S, 24, 8, 128)
                for S in (1024, 2048, 4096, 8192, 16384, 32768)]
LLAMA_8B = ("llama3.1-8b_s16k_b2", 8, 2, 16384, 32, 8, 128)

ALL = [TINY, LLAMA_1B, QWEN_1_8B] + BATCH_SWEEP + LONG_CONTEXT + [LLAMA_8B]

# More sequences than ranks: BASP reverts to data parallelism (each rank takes
# B/N whole sequences); the batch-sweep shape continued to B = 16.
DP_FALLBACK = ("llama3.2-1b_s8k_b16", 8, 16, 8192, 32, 8, 64)
EXTRA = [DP_FALLBACK]

BY_NAME = {w[0]: w for w in ALL + EXTRA}
