"""Bucket assignment of DDP gradients: which parameter goes into which flat
bucket, at which offset.

TEST INFRASTRUCTURE ONLY: part of the CPU oracle. Only the tests, the smoke
check and the CPU-baseline leg of the benchmark may import this module.

What it follows (page "DDP 与 Ring All-Reduce" (blog.vllbc.top), section 03,
parts "Bucket：把许多小梯度拼成一次集合通信" and "Overlap：桶一满就发"; page
"Day 17 数据并行 DP/DDP" (blog.ans20xx.com), part "bucket 与 overlap"):
  * many small gradients are packed into one flat bucket so that each
    collective is large;
  * buckets are filled in the reverse of the parameters' registration order,
    as an approximation of the order in which backward produces gradients;
  * the regular bucket capacity is 25 MiB (25 * 1024 * 1024 bytes); the first
    bucket's capacity is 1 MiB (1024 * 1024 bytes);
  * every rank uses the same assignment and the same bucket order.

Readings where the pages are silent or disagree (each is listed in the design
notes):
  * "capacity" is an upper limit: a tensor that would push the open bucket past
    its capacity closes it and opens the next one; a tensor larger than the
    capacity goes alone into a bucket of its own;
  * the first bucket holds the tail of the parameter list (the first gradients
    backward produces), as the reverse order implies;
  * each member starts at a multiple of V = 16 / element_size elements (one
    16-byte vector) and occupies round_up(numel, V) elements of the bucket; the
    capacity test uses these rounded sizes;
  * a bucket's length is padded with zeros to a multiple of N * V elements, so
    that its N ring chunks have equal length and start on 16-byte boundaries.
"""

MIB = 1024 * 1024
DEFAULT_CAP_BYTES = 25 * MIB          # 26,214,400
DEFAULT_FIRST_BUCKET_BYTES = 1 * MIB  # 1,048,576
VECTOR_BYTES = 16


def _round_up(x, m):
    return -(-x // m) * m


def bucket_order(n_params):
    """Parameters in the order they are bucketed: reverse registration order."""
    return reversed(range(n_params))


def bucket_capacity(index, cap_bytes, first_bucket_bytes):
    """Capacity in bytes of bucket `index`: the first bucket has its own."""
    return first_bucket_bytes if index == 0 else cap_bytes


def plan(param_numels, elem_bytes, cap_bytes=DEFAULT_CAP_BYTES,
         first_bucket_bytes=DEFAULT_FIRST_BUCKET_BYTES, world_size=1, vector_elems=None):
    """Assign parameters to buckets.

    param_numels       : element counts of the parameters, in registration order.
    elem_bytes         : 4 (fp32) or 2 (bf16): the gradients' element size, in
                         which capacities are counted.
    cap_bytes          : capacity of every bucket after the first.
    first_bucket_bytes : capacity of bucket 0.
    world_size         : N, used only for the padding of each bucket.
    vector_elems       : alignment of members and padding, in elements; by
                         default one 16-byte vector of the gradient dtype. A
                         bucket communicated in a narrower dtype (the bf16
                         compression of fp32 gradients) uses that dtype's
                         vector: 8 elements.

    Returns a list of buckets in launch order; each bucket is a dict with
      "members": list of (param_index, offset, numel), offsets in elements,
      "padded_numel": the bucket's length in elements.
    """
    if elem_bytes not in (2, 4):
        raise ValueError("elem_bytes must be 2 or 4")
    if cap_bytes <= 0 or first_bucket_bytes <= 0 or world_size < 1:
        raise ValueError("capacities and world size must be positive")
    v = VECTOR_BYTES // elem_bytes if vector_elems is None else int(vector_elems)
    if v < 1:
        raise ValueError("vector_elems must be positive")
    buckets = []
    members = []
    used = 0  # elements used in the open bucket, multiple of v

    def close():
        buckets.append({"members": members,
                        "padded_numel": _round_up(used, world_size * v)})

    for p in bucket_order(len(param_numels)):
        numel = int(param_numels[p])
        if numel < 0:
            raise ValueError("parameter sizes must be non-negative")
        slot = _round_up(numel, v)
        if members and (used + slot) * elem_bytes > bucket_capacity(len(buckets), cap_bytes,
                                                                    first_bucket_bytes):
            close()
            members, used = [], 0
        members.append((p, used, numel))
        used += slot
    if members:
        close()
    return buckets
